// align.hip -- routing permutation for the grouped GEMMs.
//
// SGLang PR #7762, review thread on run_cutlass_moe_ep_preproess: the local
// top-k ids are stable-sorted, seg_indptr holds the per-expert segment
// offsets and src2dst maps every (token, k) slot to its sorted position;
// review thread on expert_map: global ids become local ids of this rank.
// Here a pair f = t*topk + j is local when l = id[f] - expert_begin is in
// [0, E); the stable sort by l is a counting sort that visits f in
// ascending order:
//   count   -- per chunk of CH pairs, a histogram of local ids (LDS atomics);
//   scan    -- one block: counts, exclusive offsets, the per-chunk base of
//              every expert, and the m-block list;
//   scatter -- per chunk, rounds of 256 pairs in f order: the rank of a pair
//              among earlier pairs of the same expert comes from per-wave
//              64-bit lane masks in LDS and per-wave counts, so equal keys
//              keep ascending f.
// When all pairs fit one chunk the three phases run in one block (decode).
#include "common.hpp"
#include "internal.hpp"
#include "quant_block.hpp"

namespace w4a8 {

constexpr int kAlignThreads = 256;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kAlignSingle = 4096;  // up to this many pairs: one block does everything
constexpr int kAlignChunk = 1024;   // otherwise pairs per chunk (one block each)
constexpr int kMaxLocalExperts = 1024;

int64_t align_chunk_count(int64_t F)
{
    return F <= kAlignSingle ? 1 : (F + kAlignChunk - 1) / kAlignChunk;
}
size_t align_workspace_bytes(int64_t F, int64_t E)
{
    return (size_t)align_chunk_count(F) * (size_t)E * sizeof(int32_t);
}

__device__ __forceinline__ int local_id(const int32_t* ids, int64_t f, int64_t F, int64_t eb,
                                        int64_t E)
{
    if (f >= F)
        return -1;
    const int64_t l = (int64_t)ids[f] - eb;
    return (l >= 0 && l < E) ? (int)l : -1;
}

// rank of this lane among lower lanes of the wave with the same key, and the
// number of lanes with that key; keys < 0 are ignored.  masks: this wave's
// [E] 64-bit lane masks in LDS, zero on entry and on exit.  Every lane ORs
// its bit into the mask of its key, then reads it back; a wave's LDS
// operations complete in order, so the read sees every lane's bit and the
// clear (by the lowest lane of each key) follows every lane's read.  The
// cost does not depend on how many distinct keys the wave holds.
__device__ __forceinline__ void wave_rank(int key, unsigned long long* masks, int& rank, int& count)
{
    const int lane = threadIdx.x & 63;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    rank = 0;
    count = 0;
    if (key >= 0) {
        atomicOr(&masks[key], 1ull << lane);
        const unsigned long long m = masks[key];
        rank = __popcll(m & lt);
        count = __popcll(m);
        if (rank == 0)
            masks[key] = 0ull;
    }
}

// The exclusive scans of up to four arrays of n values in LDS (n <= 4 *
// kAlignThreads, a null array skipped) with one set of barriers; totals[i]
// receives array i's total.  scratch: 4 * (kAlignWaves + 1) ints.  All
// threads must call it.
__device__ void block_exclusive_scan4(int* const (&vals)[4], int n, int* scratch, int (&totals)[4])
{
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    int local[4][4], sum[4], incl[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        sum[a] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = 4 * t + i;
            local[a][i] = (vals[a] != nullptr && idx < n) ? vals[a][idx] : 0;
            sum[a] += local[a][i];
        }
        incl[a] = sum[a];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int y = __shfl_up(incl[a], o, 64);
            if (lane >= o)
                incl[a] += y;
        }
    if (lane == 63)
#pragma unroll
        for (int a = 0; a < 4; ++a)
            scratch[a * (kAlignWaves + 1) + wave] = incl[a];
    __syncthreads();
    if (t < 4) {
        int* sc = scratch + t * (kAlignWaves + 1);
        int run = 0;
        for (int w = 0; w < kAlignWaves; ++w) {
            const int c = sc[w];
            sc[w] = run;
            run += c;
        }
        sc[kAlignWaves] = run;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int* sc = scratch + a * (kAlignWaves + 1);
        int run = sc[wave] + incl[a] - sum[a];
        if (vals[a] != nullptr)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = 4 * t + i;
                if (idx < n)
                    vals[a][idx] = run;
                run += local[a][i];
            }
        totals[a] = sc[kAlignWaves];
    }
    __syncthreads();
}

// counts[] (LDS, E entries) -> offsets, counts and block list(s) in global
// memory; leaves the exclusive offsets in counts_lds.  With two lists
// (o.block_expert2 != null) an expert's blocks go to the first list (block_m
// rows) when it has at most o.small_rows pairs, else to the second
// (o.block_m2 rows).  Returns true (in every thread) when the local pairs
// exceed o.max_pairs: then the offsets, block counts and block_start are
// zero, no block is listed, and the caller must scatter no pair.  All
// threads call it.
// Rows a block-tiled wave pair computes for a tile of r rows: each 80-row
// half is computed in whole 16-row slices.
__device__ __forceinline__ float tile_rows16(int r)
{
    const int h0 = min(r, kTileRows / 2), h1 = max(r - kTileRows / 2, 0);
    return 16.0f * (float)((h0 + 15) / 16 + (h1 + 15) / 16);
}

// Predicted us of the slowest workgroup of each of the two block-tiled
// launches (gate_up, down): nb m-blocks (bstart [E] their exclusive prefix
// per expert, off [E] the experts' first rows, P rows in all); launch k has
// nbn[k] tiles per m-block and wgs[k] <= kAlignThreads workgroups walking the
// tiles in the launchers' order (tile L = expert major, then weight block,
// m-block fastest; XCD x = w % 8 takes the x-th eighth, its workgroups every
// (wgs / 8)-th tile of it).  Each expert's tiles are split over threads,
// which add every tile's cost to its workgroup's sum in LDS (wg_cost: 2 x
// kAlignThreads floats; red: 2 ints of LDS).  All threads call it.
__device__ void tiled_launches_us(const PathCost& c, const int* bstart, const int* off, int P, int64_t E,
                                  int nb, float* wg_cost, int* red, float (&us)[2])
{
    const int t = threadIdx.x;
    const int nbn[2] = {c.nbn_gu, c.nbn_dn}, wgs[2] = {c.wgs_gu, c.wgs_dn};
    const float groups[2] = {c.groups_gu, c.groups_dn}, c0[2] = {c.gu0, c.dn0}, c1[2] = {c.gu1, c.dn1};
    wg_cost[t] = 0.0f;
    wg_cost[kAlignThreads + t] = 0.0f;
    if (t < 2)
        red[t] = 0;
    __syncthreads();
    const int parts = E < kAlignThreads ? kAlignThreads / (int)E : 1;  // threads per expert
    for (int i = t; i < E * parts; i += kAlignThreads) {
        const int e = i / parts, part = i - e * parts;
        const int bs = bstart[e];
        const int nbe = (e + 1 < E ? bstart[e + 1] : nb) - bs;
        if (nbe == 0 || part >= nbe * max(nbn[0], nbn[1]))
            continue;
        const int cnt = (e + 1 < E ? off[e + 1] : P) - off[e];
        const float rows_full = tile_rows16(kTileRows);
        const float rows_last = tile_rows16(cnt - kTileRows * (nbe - 1));
        const int step_m = parts % nbe;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int n = nbe * nbn[k];
            if (part >= n)
                continue;
            const int total = nb * nbn[k], per_xcd = (total + 7) >> 3, stride = wgs[k] >> 3;
            const float full = groups[k] * (c0[k] + c1[k] * rows_full);
            const float last = groups[k] * (c0[k] + c1[k] * rows_last);
            float* acc = wg_cost + k * kAlignThreads;
            // tile L = bs * nbn + j (j = part, part + parts, ...): its XCD x,
            // its place tx in that XCD's range and its workgroup's slot tm =
            // tx % stride, and its m-block mb = j % nbe, all stepped without a
            // division per tile (the block runs one wave per SIMD, so a
            // division chain per tile would sit on the align's critical path)
            const int L = bs * nbn[k] + part;
            int x = L / per_xcd, tx = L - x * per_xcd, tm = tx % stride, mb = part % nbe;
            const int step_t = parts % stride;
            for (int j = part;;) {
                atomicAdd(&acc[(tm << 3) | x], mb == nbe - 1 ? last : full);
                j += parts;
                if (j >= n)
                    break;
                mb += step_m;
                if (mb >= nbe)
                    mb -= nbe;
                tx += parts;
                if (tx >= per_xcd) {
                    while (tx >= per_xcd) {
                        tx -= per_xcd;
                        ++x;
                    }
                    tm = tx % stride;
                } else {
                    tm += step_t;
                    if (tm >= stride)
                        tm -= stride;
                }
            }
        }
    }
    __syncthreads();
    // the slowest workgroup of each launch: a max over the wave by shuffles,
    // then over the waves (256 atomics on one LDS word measured ~2.5 us)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        float m = t < wgs[k] ? wg_cost[k * kAlignThreads + t] : 0.0f;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o, 64));
        if ((t & 63) == 0)
            atomicMax(&red[k], __float_as_int(m));  // non-negative floats order like their bits
    }
    __syncthreads();
    us[0] = __int_as_float(red[0]);
    us[1] = __int_as_float(red[1]);
    __syncthreads();
}

// Predicted us of the two GEMMs on the block-tiled path minus the skinny one
// (see PathCost): < 0 picks the block-tiled kernels.  bstart / off /
// wg_cost / red: LDS, as in tiled_launches_us.  All threads call it.
__device__ float tiled_minus_skinny(const PathCost& c, const int* bstart, const int* off, int P,
                                    int64_t E, int nb_skinny, int nb_tiled, float* wg_cost, int* red)
{
    float us[2];
    tiled_launches_us(c, bstart, off, P, E, nb_tiled, wg_cost, red, us);
    return us[0] + us[1] - (c.skinny_fixed_us + (float)nb_skinny * c.skinny_block_us);
}

__device__ bool finish_scan(int* counts_lds, int* tmp_lds, int* tmp2_lds, int* tmp3_lds, int* scratch,
                            float* wg_cost, int64_t E, int64_t block_m, const AlignOut& o)
{
    const int t = threadIdx.x;
    const bool dual = o.block_expert2 != nullptr;
    const bool choose = o.path != nullptr;  // also the kTileRows-row list
    if (t == 0 && o.barrier != nullptr)
        o.barrier[0] = 0;
    for (int e = t; e < E; e += kAlignThreads) {
        const int c = counts_lds[e];  // written out after the scans (no store pending at their barriers)
        const bool second = dual && c > o.small_rows;
        tmp_lds[e] = second ? 0 : (int)((c + block_m - 1) / block_m);  // m-blocks of expert e
        tmp2_lds[e] = second ? (c + o.block_m2 - 1) / o.block_m2 : 0;
        tmp3_lds[e] = choose ? (c + kTileRows - 1) / kTileRows : 0;
    }
    __syncthreads();
    int tot[4];
    int* const arrs[4] = {counts_lds, tmp_lds, dual ? tmp2_lds : nullptr, choose ? tmp3_lds : nullptr};
    block_exclusive_scan4(arrs, (int)E, scratch, tot);
    const int P = tot[0], nb = tot[1], nb2 = tot[2], nb3 = tot[3];
    const bool over = o.max_pairs > 0 && P > o.max_pairs;  // P is the same in every thread
    // (the scans leave the exclusive prefixes in counts_lds and tmp3_lds)
    const int path = !choose ? o.static_path
                     : over  ? 0
                             : (tiled_minus_skinny(o.cost, tmp3_lds, counts_lds, P, E, nb + nb2, nb3, wg_cost, scratch) < 0.0f
                                    ? 1 : 0);
    // block_start belongs to the list the block-tiled kernels read
    const int* bs_lds = choose ? tmp3_lds : tmp_lds;
    const int nbs = choose ? nb3 : nb;
    for (int e = t; e < E; e += kAlignThreads) {
        o.offsets[e] = over ? 0 : counts_lds[e];
        o.counts[e] = (e + 1 < E ? counts_lds[e + 1] : P) - counts_lds[e];
    }
    if (t == 0) {
        o.offsets[E] = over ? 0 : P;
        *o.num_blocks = over ? 0 : nb;
        if (dual)
            *o.num_blocks2 = over ? 0 : nb2;
        if (choose) {
            *o.num_blocks3 = over ? 0 : nb3;
            *o.path = path;
        }
        if (o.block_start != nullptr)
            o.block_start[E] = over ? 0 : nbs;
        if (o.pairs_out != nullptr) {
            o.pairs_out[0] = P;
            o.pairs_out[1] = path;
        }
    }
    if (o.block_start != nullptr)
        for (int e = t; e < E; e += kAlignThreads)
            o.block_start[e] = over ? 0 : bs_lds[e];
    if (choose && !over) {
        for (int e = t; e < E; e += kAlignThreads) {
            const int first = tmp3_lds[e];
            const int last = (e + 1 < E) ? tmp3_lds[e + 1] : nb3;
            for (int b = first; b < last; ++b)
                o.block_row3[b] = counts_lds[e] + (b - first) * kTileRows;
        }
    }
    if (o.block_expert != nullptr && !over) {
        for (int e = t; e < E; e += kAlignThreads) {
            const int first = tmp_lds[e];
            const int last = (e + 1 < E) ? tmp_lds[e + 1] : nb;
            for (int b = first; b < last; ++b) {
                o.block_expert[b] = e;
                o.block_row[b] = counts_lds[e] + (int)((b - first) * block_m);
            }
            if (dual) {
                const int first2 = tmp2_lds[e];
                const int last2 = (e + 1 < E) ? tmp2_lds[e + 1] : nb2;
                for (int b = first2; b < last2; ++b) {
                    o.block_expert2[b] = e;
                    o.block_row2[b] = counts_lds[e] + (b - first2) * o.block_m2;
                }
            }
        }
    }
    __syncthreads();
    return over;
}

// the local ids of pairs f0 + r * kAlignThreads + t, r < R (-1 past f1),
// loaded once: every round below uses registers.  All R loads are issued
// before any is used (addresses clamped into [f0, f1), f1 > f0).
template <int R>
__device__ __forceinline__ void load_keys(const int32_t* ids, int64_t f0, int64_t f1, int64_t eb,
                                          int64_t E, int (&keys)[R])
{
    int32_t raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t f = f0 + (int64_t)r * kAlignThreads + threadIdx.x;
        raw[r] = ids[f < f1 ? f : f1 - 1];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t f = f0 + (int64_t)r * kAlignThreads + threadIdx.x;
        const int64_t l = (int64_t)raw[r] - eb;
        keys[r] = (f < f1 && l >= 0 && l < E) ? (int)l : -1;
    }
}

// scatter one chunk [f0, f1) (at most R rounds of kAlignThreads pairs, keys
// from load_keys) given the running base position of every expert (LDS);
// wcnt ([kAlignWaves][E] ints) and masks ([kAlignWaves][E] lane masks) are
// zero on entry and on exit.
template <int R>
__device__ void scatter_chunk(const int (&keys)[R], int64_t f0, int64_t f1, int64_t E, int* base,
                              int* wcnt, unsigned long long* masks, const AlignOut& o)
{
    const int t = threadIdx.x, wave = t >> 6;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t r0 = f0 + (int64_t)r * kAlignThreads;
        if (r0 >= f1)
            break;
        const int64_t f = r0 + t;
        const int key = keys[r];
        int rank, count;
        wave_rank(key, masks + wave * E, rank, count);
        const bool leader = key >= 0 && rank == 0;
        if (leader)
            wcnt[wave * E + key] = count;
        __syncthreads();
        if (key >= 0) {
            int pos = base[key] + rank;
            for (int w = 0; w < wave; ++w)
                pos += wcnt[w * E + key];
            o.sorted[pos] = (int32_t)f;
            o.src2dst[f] = pos;
        } else if (f < f1) {
            o.src2dst[f] = -1;
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&base[key], count);
            wcnt[wave * E + key] = 0;
        }
        __syncthreads();
    }
}

struct AlignLds {
    int a[kMaxLocalExperts];
    int b[kMaxLocalExperts];
    int c[kMaxLocalExperts];
    int d[kMaxLocalExperts];
    float wg_cost[2 * kAlignThreads];
    int wcnt[kAlignWaves * kMaxLocalExperts];
    int scratch[4 * (kAlignWaves + 1)];
};
constexpr int kSingleRounds = kAlignSingle / kAlignThreads;  // 16
constexpr int kChunkRounds = kAlignChunk / kAlignThreads;    // 4
// the lane masks of wave_rank, [kAlignWaves][E]: dynamic LDS of the launch
extern __shared__ unsigned long long align_masks[];
size_t align_mask_bytes(int64_t E)
{
    return (size_t)kAlignWaves * (size_t)E * sizeof(unsigned long long);
}

// everything in one block (F <= kAlignSingle).  Wave w owns the pairs
// [w * seg, (w + 1) * seg) in 64-lane rounds, so f order is (wave, round,
// lane) order and a pair's place among the pairs of its expert is: the
// expert's offset + the expert's pairs in earlier waves + in this wave's
// earlier rounds + its rank in its round.  The waves count their own
// pairs per expert without any barrier (a wave's LDS operations complete in
// order); one barrier then joins the counts, and the scan and the per-wave
// bases follow before each lane writes its pairs.
__device__ __forceinline__ void align_single_body(const int32_t* __restrict__ ids, int64_t F,
                                                  int64_t eb, int64_t E, int64_t block_m,
                                                  const AlignOut& o, AlignLds& L)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t seg = ((F + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64;  // <= 1024
    const int64_t f0 = wave * seg;
    // every load issued before any is used (a load per round behind a
    // branch made them wait one by one: ~0.8 us per round)
    int32_t raw[kSingleRounds];
#pragma unroll
    for (int r = 0; r < kSingleRounds; ++r) {
        const int64_t f = f0 + r * 64 + lane;
        raw[r] = ids[f < F ? f : F - 1];
    }
    int keys[kSingleRounds];
#pragma unroll
    for (int r = 0; r < kSingleRounds; ++r) {
        const int64_t f = f0 + r * 64 + lane;
        const int64_t l = (int64_t)raw[r] - eb;
        keys[r] = (r * 64 < seg && f < F && l >= 0 && l < E) ? (int)l : -1;
    }
    for (int i = t; i < kAlignWaves * E; i += kAlignThreads) {
        L.wcnt[i] = 0;
        align_masks[i] = 0ull;
    }
    __syncthreads();
    // this wave's pairs per expert, and each lane's place among them
    int* cnt = L.wcnt + wave * E;
    int pos[kSingleRounds];
#pragma unroll
    for (int r = 0; r < kSingleRounds; ++r) {
        pos[r] = 0;
        if (r * 64 >= seg)
            break;
        int rank, count;
        wave_rank(keys[r], align_masks + wave * E, rank, count);
        if (keys[r] >= 0) {
            pos[r] = cnt[keys[r]] + rank;
            if (rank == 0)
                cnt[keys[r]] += count;  // after every lane's read: in order
        }
    }
    __syncthreads();
    for (int e = t; e < E; e += kAlignThreads) {
        int c = 0;
        for (int w = 0; w < kAlignWaves; ++w)
            c += L.wcnt[w * E + e];
        L.a[e] = c;
    }
    __syncthreads();
    // L.a now holds the offsets
    const bool over = finish_scan(L.a, L.b, L.c, L.d, L.scratch, L.wg_cost, E, block_m, o);
    for (int e = t; e < E; e += kAlignThreads) {  // the waves' bases per expert
        int run = L.a[e];
        for (int w = 0; w < kAlignWaves; ++w) {
            const int c = L.wcnt[w * E + e];
            L.wcnt[w * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSingleRounds; ++r) {
        if (r * 64 >= seg)
            break;
        const int64_t f = f0 + r * 64 + lane;
        if (f >= F)
            break;
        if (keys[r] >= 0 && !over) {  // over capacity: no pair is placed, src2dst = -1
            const int p = cnt[keys[r]] + pos[r];
            o.sorted[p] = (int32_t)f;
            o.src2dst[f] = p;
        } else {
            o.src2dst[f] = -1;
        }
    }
}

__global__ __launch_bounds__(kAlignThreads) void align_single_kernel(const int32_t* __restrict__ ids,
                                                                     int64_t F, int64_t eb,
                                                                     int64_t E, int64_t block_m,
                                                                     AlignOut o)
{
    __shared__ AlignLds L;
    align_single_body(ids, F, eb, E, block_m, o, L);
}

// The routing permutation and the activation quantisation are independent:
// one launch does both.  Block 0 runs the single-block align; blocks 1..
// quantise (mode 1).
__global__ __launch_bounds__(kAlignThreads) void align_quant_kernel(
    const int32_t* __restrict__ ids, int64_t F, int64_t eb, int64_t E, int64_t block_m, AlignOut o,
    const uint16_t* __restrict__ x, int64_t M,
    int64_t K, int64_t ldx, uint8_t* __restrict__ q, float2* __restrict__ side,
    const float* __restrict__ fixed_scale)
{
    __shared__ AlignLds L;
    if (blockIdx.x == 0) {
        align_single_body(ids, F, eb, E, block_m, o, L);
        return;
    }
    quant_block<1>(x, M, K, ldx, q, nullptr, side, (int64_t)blockIdx.x - 1, fixed_scale);
}

// a block of the quantisation that rides along with the chunked align:
// quantisation block qb of job qj
__device__ __forceinline__ void quant_rider(const QuantJob& qj, int64_t qb)
{
    quant_block<1>(qj.x, qj.M, qj.K, qj.ldx, qj.q, nullptr, qj.side, qb, qj.fixed_scale);
}

// blocks [0, nchunks) count, blocks nchunks.. quantise blocks [0, q_count) of qj
__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(const int32_t* __restrict__ ids,
                                                                    int64_t F, int64_t eb,
                                                                    int64_t E,
                                                                    int32_t* __restrict__ hist,
                                                                    QuantJob qj)
{
    __shared__ int cnt[kMaxLocalExperts];
    const int64_t nchunks = (F + kAlignChunk - 1) / kAlignChunk;
    if ((int64_t)blockIdx.x >= nchunks) {
        quant_rider(qj, (int64_t)blockIdx.x - nchunks);
        return;
    }
    const int t = threadIdx.x;
    const int64_t f0 = (int64_t)blockIdx.x * kAlignChunk;
    const int64_t f1 = f0 + kAlignChunk < F ? f0 + kAlignChunk : F;
    int keys[kChunkRounds];
    load_keys(ids, f0, f1, eb, E, keys);  // the loads overlap the clearing below
    for (int e = t; e < E; e += kAlignThreads)
        cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kChunkRounds; ++r)
        if (keys[r] >= 0)
            atomicAdd(&cnt[keys[r]], 1);
    __syncthreads();
    for (int e = t; e < E; e += kAlignThreads)
        hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(int32_t* __restrict__ hist,
                                                                   int64_t nchunks, int64_t E,
                                                                   int64_t block_m, AlignOut o)
{
    // hist[c * E + e] = pairs of local expert e in chunk c  ->  the sorted
    // position of the first of them.  Two levels, so that every thread has
    // work: thread i = g * E + e sums expert e over chunk group g (ng groups
    // of cpg consecutive chunks; one group when E exceeds the block), the
    // group sums are prefixed per expert in LDS, the experts' totals go
    // through finish_scan, and each thread writes its group's running bases.
    __shared__ AlignLds L;
    __shared__ int part[kMaxLocalExperts];  // [g][e]: group sums, then their exclusive prefix
    const int t = threadIdx.x;
    const int ng = E <= kAlignThreads ? kAlignThreads / (int)E : 1;
    const int64_t cpg = (nchunks + ng - 1) / ng;
    constexpr int kBatch = 8;  // counts read per batch, so the loads overlap
    for (int i = t; i < ng * E; i += kAlignThreads) {
        const int g = i / (int)E, e = i - g * (int)E;
        const int64_t c0 = g * cpg, c1 = c0 + cpg < nchunks ? c0 + cpg : nchunks;
        int run = 0;
        for (int64_t c = c0; c < c1; c += kBatch) {
            int h[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                h[j] = c + j < c1 ? hist[(c + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                run += h[j];
        }
        part[i] = run;
    }
    __syncthreads();
    for (int e = t; e < E; e += kAlignThreads) {
        int run = 0;
        for (int g = 0; g < ng; ++g) {
            const int v = part[g * E + e];
            part[g * E + e] = run;
            run += v;
        }
        L.a[e] = run;
    }
    __syncthreads();
    finish_scan(L.a, L.b, L.c, L.d, L.scratch, L.wg_cost, E, block_m, o);  // L.a now holds the experts' offsets
    for (int i = t; i < ng * E; i += kAlignThreads) {
        const int g = i / (int)E, e = i - g * (int)E;
        const int64_t c0 = g * cpg, c1 = c0 + cpg < nchunks ? c0 + cpg : nchunks;
        int run = L.a[e] + part[i];
        for (int64_t c = c0; c < c1; c += kBatch) {
            int h[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                h[j] = c + j < c1 ? hist[(c + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (c + j < c1)
                    hist[(c + j) * E + e] = run;
                run += h[j];
            }
        }
    }
}

// blocks [0, nchunks) scatter, blocks nchunks.. quantise blocks q_first.. of qj
__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(const int32_t* __restrict__ ids,
                                                                      int64_t F, int64_t eb,
                                                                      int64_t E,
                                                                      const int32_t* __restrict__ hist,
                                                                      AlignOut o, QuantJob qj,
                                                                      int64_t q_first)
{
    __shared__ int base[kMaxLocalExperts];
    __shared__ int wcnt[kAlignWaves * kMaxLocalExperts];
    const int64_t nchunks = (F + kAlignChunk - 1) / kAlignChunk;
    if ((int64_t)blockIdx.x >= nchunks) {
        quant_rider(qj, q_first + (int64_t)blockIdx.x - nchunks);
        return;
    }
    const int t = threadIdx.x;
    const int64_t f0 = (int64_t)blockIdx.x * kAlignChunk;
    const int64_t f1 = f0 + kAlignChunk < F ? f0 + kAlignChunk : F;
    int keys[kChunkRounds];
    load_keys(ids, f0, f1, eb, E, keys);
    // offsets[E] == 0: no local pair, or more than the buffers hold (the scan
    // then zeroed the offsets); either way no pair is placed
    if (o.offsets[E] == 0) {
#pragma unroll
        for (int r = 0; r < kChunkRounds; ++r)
            keys[r] = -1;
    }
    for (int e = t; e < E; e += kAlignThreads)
        base[e] = hist[(int64_t)blockIdx.x * E + e];
    for (int i = t; i < kAlignWaves * E; i += kAlignThreads) {
        wcnt[i] = 0;
        align_masks[i] = 0ull;
    }
    __syncthreads();
    scatter_chunk(keys, f0, f1, E, base, wcnt, align_masks, o);
}

hipError_t launch_align_quant(const int32_t* ids, int64_t T, int64_t topk, int64_t expert_begin,
                              int64_t E, int64_t block_m, const AlignOut& o, const uint16_t* x,
                              int64_t H, uint8_t* q,
                              float2* side, const float* fixed_scale, hipStream_t s)
{
    const int64_t F = T * topk;
    const int64_t qblocks = (T * (H / kGroup) + 15) / 16;
    hipLaunchKernelGGL(align_quant_kernel, dim3((unsigned)(1 + qblocks)), dim3(kAlignThreads),
                       (unsigned)align_mask_bytes(E), s,
                       ids, F, expert_begin, E, block_m, o, x, T, H, H, q, side,
                       fixed_scale);
    return hipGetLastError();
}

hipError_t launch_align(const int32_t* ids, int64_t T, int64_t topk, int64_t expert_begin,
                        int64_t E, int64_t block_m, const AlignOut& o, void* ws, hipStream_t s,
                        const QuantJob& qj)
{
    const int64_t F = T * topk;
    const int64_t nchunks = align_chunk_count(F);
    if (nchunks == 1) {  // (a quantisation job goes with launch_align_quant instead)
        hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(kAlignThreads),
                           (unsigned)align_mask_bytes(E), s, ids, F, expert_begin, E, block_m, o);
        return hipGetLastError();
    }
    // The quantisation's blocks ride along, half with the count launch and
    // half with the scatter launch, so that both short launches overlap it
    // (T=4096, top-8: align and quantisation 42 us apart, 36 us together).
    const int64_t qblocks = qj.x != nullptr ? (qj.M * (qj.K / kGroup) + 15) / 16 : 0;
    const int64_t q1 = (qblocks + 1) / 2, q2 = qblocks - q1;
    int32_t* hist = (int32_t*)ws;
    hipLaunchKernelGGL(align_count_kernel, dim3((unsigned)(nchunks + q1)), dim3(kAlignThreads), 0, s,
                       ids, F, expert_begin, E, hist, qj);
    hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kAlignThreads), 0, s, hist, nchunks, E,
                       block_m, o);
    hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)(nchunks + q2)), dim3(kAlignThreads),
                       (unsigned)align_mask_bytes(E), s, ids, F, expert_begin, E, hist, o, qj, q1);
    return hipGetLastError();
}

} // namespace w4a8
