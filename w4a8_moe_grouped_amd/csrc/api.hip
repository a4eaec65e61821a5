// api.hip -- the C ABI of libw4a8 (declared and documented in include/w4a8.h).
//
// Host-side only: argument validation (before any HIP call), workspace
// planning and the launch sequence of each export.  No allocation, no
// synchronisation, no state between calls.
#include "w4a8.h"

#include "internal.hpp"

#include <algorithm>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int64_t kMaxLocalExperts = 1024;
constexpr size_t kAlign = 256;

inline size_t round_up(size_t x)
{
    return (x + kAlign - 1) / kAlign * kAlign;
}
inline bool aligned16(const void* p)
{
    return ((uintptr_t)p & 15u) == 0;
}

// A bump allocator over the caller's workspace (or over nothing, to size it).
struct Carve {
    char* base;
    size_t used = 0;
    explicit Carve(void* b) : base((char*)b) {}
    template <typename T>
    T* take(size_t count)
    {
        T* p = base ? (T*)(base + used) : nullptr;
        used += round_up(count * sizeof(T));
        return p;
    }
};

// rows per m-block for the skinny grouped GEMM: from the pairs each local
// expert would get if every pair were local (the host does not see the routing)
int pick_block_m(int64_t pairs, int64_t experts)
{
    const int64_t per = experts > 0 ? (pairs + experts - 1) / experts : pairs;
    if (per <= 16)
        return 16;
    if (per <= 32)
        return 32;
    return 64;
}

int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

// Between the decode regime (at most 16 pairs per expert: 16-row blocks) and
// the block-tiled one, the block height is chosen per expert on the device,
// from the counts: the align writes two m-block lists, blocks of 16 rows for
// experts with at most 16 pairs and of 32 rows for the others, and the
// skinny GEMM runs once over each.  The host's figure T*topk/E_l counts every
// pair as local; on an expert-parallel share only E_l/E of them are (8x
// fewer rows), and skewed routing puts 5 rows on one expert and 250 on the
// next.  Measured per fused call against one height for all experts (32 of
// 256 experts, top-8; 16 / 32 / 64-row blocks everywhere): 128 tokens 133 /
// 152 / 202 us, 256 tokens 172 / 179 / 222, 512 tokens 202 / 193 / 244,
// Zipf routing with rank = expert id 470 / 401 / 443.
constexpr int kSmallExpertRows = 16;
constexpr int kLargeBlockRows = 32;
bool use_two_lists(int64_t pairs, int64_t experts)
{
    return pairs > 16 * experts;
}

// Many rows per expert: the block-tiled GEMM (160-row m-blocks, weights
// reused across the rows of an m-block from LDS) beats streaming the weights
// once per small m-block.  Decided from the pairs per expert if every pair
// were local, like pick_block_m.
constexpr int64_t kTilePairsPerExpert = 256;
bool use_tile(int64_t pairs, int64_t experts)
{
    return pairs >= kTilePairsPerExpert * experts;
}

// With a caller's bound on the local pairs (w4a8_fused_moe_bounded) the
// host's estimate is close to the real count rather than 8x above it (on an
// expert-parallel share of 32 of 256 experts the rules above see T*topk/E_l
// where the experts get about T*topk/256), so the path is chosen from real
// rows per local expert.  Measured per call with the bound = pairs + 8 (32
// of 256 experts, top-8, H = 7168, I = 2048; two-list skinny vs block-tiled):
// ~16 rows per expert 192 vs 330 us, ~32 rows 296 vs 336, ~64 rows 454 vs
// 406; Zipf routing with rank = expert id (61 rows per expert on average,
// 5 to 252) 381 vs 632.
constexpr int64_t kBoundedTileRows = 64;     // block-tiled from this many rows per expert
constexpr int64_t kBoundedTwoListRows = 2;   // per-expert 16 / 32-row blocks above this

// Between these regimes the counts decide (DeepGEMM PR #53 commit notes: an
// expected-cost argmin over the per-expert token counts replaces hand-set
// boundaries; there the counts are Poisson expectations, here the align has
// the real ones).  The align writes the block-tiled path's m-block list
// beside the two skinny lists and predicts both paths' GEMM time;
// both GEMM kernels are launched and the one not chosen exits at once.
// Fitted by least squares on MI355X (32 local experts, top-8, H = 7168,
// I = 2048; uniform routing at 8 to 128 rows per expert, two Zipf routings,
// T = 4096): the two skinny GEMMs cost 39.8 us plus, per m-block, one
// expert's weights (1.5*H*I bytes) at 4.95 TB/s; a 160 x 256 tile costs per
// 128-K group 0.815 us + 0.01327 us per computed row in gate_up and
// 0.776 + 0.00833 in the down GEMM, summed over the tiles of the slowest
// workgroup (predictions within 3% of the tiled and 8% of the skinny times
// measured; the faster path picked on all eight workloads).
// The choice is offered while the skinny lists stay below kChoiceMaxBlocks
// m-blocks (the launch not taken then costs a few us).
constexpr int64_t kChoiceMaxBlocks = 4096;
w4a8::PathCost path_cost(int64_t H, int64_t I, int64_t nb3_max)
{
    w4a8::PathCost c;
    c.skinny_fixed_us = 39.8f;
    c.skinny_block_us = (float)(1.5 * (double)H * (double)I / 4.95e6);
    c.groups_gu = (float)(H / W4A8_GROUP);
    c.groups_dn = (float)(I / W4A8_GROUP);
    c.nbn_gu = (int32_t)(I / W4A8_GROUP);
    c.nbn_dn = (int32_t)((H + 255) / 256);
    // the align sums the cost of at most 256 workgroups per launch (one LDS
    // slot per thread); a GPU with more CUs is modelled with 256
    const int64_t wgs_cap = 256;
    c.wgs_gu = (int32_t)std::min(w4a8::tile_launch_workgroups(c.nbn_gu * nb3_max), wgs_cap);
    c.wgs_dn = (int32_t)std::min(w4a8::tile_launch_workgroups(c.nbn_dn * nb3_max), wgs_cap);
    c.gu0 = 0.815f;
    c.gu1 = 0.01327f;
    c.dn0 = 0.776f;
    c.dn1 = 0.00833f;
    return c;
}

// The fused forward's workspace.  P is unknown on the host, so every
// per-pair buffer is sized for `cap` pairs: F = T*topk, or the caller's bound
// on the local pairs (w4a8_fused_moe_bounded), which the align enforces.
struct MoePlan {
    bool tile;
    bool two_lists;  // per-expert 16 / 32-row blocks (see use_two_lists)
    bool choose;     // two lists and the block-tiled list, the path chosen on the device
    int block_m;
    int64_t F, cap, nb_max, nb2_max, nb3_max;
    w4a8::AlignOut al;
    void* align_ws;
    uint8_t* qa;
    float2* qa_side;
    uint8_t* qh;
    float2* qh_side;
    float* y2;
    int32_t* block_start;
};

// down_group < 128 (the finer activation recipes) runs on the skinny kernel.
// max_pairs: the caller's bound on the local pairs (0: none).  The path and
// block heights are chosen from the bounded count, the closer estimate.
// persistent: the single-launch tail (block-tiled kernels at any size, plus
// its grid-barrier counter).
size_t plan_moe(void* ws, int64_t T, int64_t H, int64_t topk, int64_t E, int64_t I, MoePlan& p,
                int down_group = W4A8_GROUP, int64_t max_pairs = 0, bool persistent = false)
{
    Carve c(ws);
    p.F = T * topk;
    p.cap = max_pairs > 0 && max_pairs < p.F ? max_pairs : p.F;
    const bool bounded = p.cap < p.F;
    // the skinny lists' m-block bound if the two lists were used
    const int64_t lists_max = ceil_div(p.cap, kSmallExpertRows) + ceil_div(p.cap, kLargeBlockRows) + 2 * E;
    if (down_group != W4A8_GROUP) {
        p.tile = p.two_lists = p.choose = false;
    } else if (persistent) {
        p.tile = true;
        p.two_lists = p.choose = false;
    } else if (bounded) {
        // the counts decide above 2 rows per expert while the skinny grid stays small
        p.choose = p.cap > kBoundedTwoListRows * E && lists_max <= kChoiceMaxBlocks;
        p.tile = !p.choose && p.cap >= kBoundedTileRows * E;
        p.two_lists = p.choose || (!p.tile && p.cap > kBoundedTwoListRows * E);
    } else {
        // between the decode and the prefill rule the counts decide
        p.tile = use_tile(p.F, E);
        p.two_lists = !p.tile && use_two_lists(p.F, E);
        p.choose = p.two_lists && lists_max <= kChoiceMaxBlocks;
    }
    p.block_m = p.tile ? w4a8::kTileRows : p.two_lists ? kSmallExpertRows : pick_block_m(p.cap, E);
    p.nb_max = ceil_div(p.cap, p.block_m) + E;
    p.nb2_max = p.two_lists ? ceil_div(p.cap, kLargeBlockRows) + E : 0;
    p.nb3_max = p.choose ? ceil_div(p.cap, w4a8::kTileRows) + E : 0;
    p.al.max_pairs = p.cap < p.F ? (int32_t)p.cap : 0;
    p.al.pairs_out = nullptr;
    p.al.static_path = p.tile ? 1 : 0;
    p.al.cost = p.choose ? path_cost(H, I, p.nb3_max) : w4a8::PathCost{};
    p.al.counts = c.take<int32_t>(E);
    p.al.offsets = c.take<int32_t>(E + 1);
    p.al.sorted = c.take<int32_t>(p.cap);
    p.al.src2dst = c.take<int32_t>(p.F);
    p.al.block_expert = c.take<int32_t>(p.nb_max);
    p.al.block_row = c.take<int32_t>(p.nb_max);
    p.al.num_blocks = c.take<int32_t>(1);
    p.align_ws = c.take<char>(w4a8::align_workspace_bytes(p.F, E));
    p.qa = c.take<uint8_t>(T * H);  // fp8 gate_up operand
    p.qa_side = c.take<float2>(T * (H / W4A8_GROUP));
    p.qh = c.take<uint8_t>(p.cap * I);
    // side data of the requantised intermediate: room for the finest recipe
    // (one block per 32 K), whatever the call uses
    p.qh_side = c.take<float2>(p.cap * (I / 32));
    p.y2 = c.take<float>(p.cap * H);
    p.al.block_start = c.take<int32_t>(E + 1);
    p.block_start = p.al.block_start;
    p.al.block_expert2 = p.two_lists ? c.take<int32_t>(p.nb2_max) : nullptr;
    p.al.block_row2 = p.two_lists ? c.take<int32_t>(p.nb2_max) : nullptr;
    p.al.num_blocks2 = p.two_lists ? c.take<int32_t>(1) : nullptr;
    p.al.small_rows = kSmallExpertRows;
    p.al.block_m2 = kLargeBlockRows;
    p.al.block_row3 = p.choose ? c.take<int32_t>(p.nb3_max) : nullptr;
    p.al.num_blocks3 = p.choose ? c.take<int32_t>(1) : nullptr;
    p.al.path = p.choose ? c.take<int32_t>(1) : nullptr;
    p.al.barrier = persistent ? c.take<int32_t>(1) : nullptr;
    return c.used;
}

// The dense GEMM's launch (dense.hip): workgroups of 128 rows x 64 weight
// rows; K is cut into slices of at most 16 groups, and further while fewer
// than ~256 workgroups would run (M = 128, N = 2048: 32 column blocks, 8
// slices of 7 groups), the slices' fp32 partial sums added in slice order by
// a second kernel.
constexpr int64_t kGemmTargetWgs = 256;
int32_t gemm_split_groups(int64_t M, int64_t K, int64_t N)
{
    const int64_t G = K / W4A8_GROUP;
    const int64_t tiles = ceil_div(N, 64) * ceil_div(M, 128);
    const int64_t want = tiles >= kGemmTargetWgs ? 1 : ceil_div(kGemmTargetWgs, tiles);
    const int64_t gps = ceil_div(G, want);
    const int64_t cap = w4a8::dense_max_split_groups();
    return (int32_t)(gps < cap ? gps : cap);
}

size_t plan_gemm(void* ws, int64_t M, int64_t K, int64_t N, float** part)
{
    Carve c(ws);
    const int64_t splits = ceil_div(K / W4A8_GROUP, gemm_split_groups(M, K, N));
    *part = splits > 1 ? c.take<float>((size_t)splits * M * N) : nullptr;
    return c.used;
}

// The GEMM kernels address their operands through buffer resources, whose
// extent and per-lane offsets are 32-bit: every byte range one resource
// covers (activation rows x K, one expert's weights or scales) must stay
// below 2^32.  The skinny GEMM puts m-blocks on grid.y (at most 65535).
constexpr int64_t kRangeLimit = (int64_t)1 << 32;
constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxPersistentH = (int64_t)1 << 24;
inline bool below_u32(int64_t bytes)
{
    return bytes >= 0 && bytes < kRangeLimit;
}
// products of non-negative sizes without int64 overflow (limit 2^62)
inline int64_t mul_sat(int64_t a, int64_t b)
{
    const int64_t cap = (int64_t)1 << 62;
    if (a <= 0 || b <= 0)
        return 0;
    return a > cap / b ? cap : a * b;
}

int check_workspace(void* ws, size_t* bytes, size_t need)
{
    if (bytes == nullptr)
        return W4A8_ERR_INVALID_ARG;
    if (ws == nullptr) {
        *bytes = need;
        return W4A8_OK;
    }
    if (*bytes < need)
        return W4A8_ERR_WORKSPACE;
    if (!aligned16(ws))
        return W4A8_ERR_UNSUPPORTED;
    return -1;  // proceed
}

inline int hip_status(hipError_t e)
{
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

// events armed by w4a8_fused_moe_stage_events for the next call on this
// thread (the handles are copied, the caller's array may go away)
thread_local void* t_stage_events[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
thread_local bool t_stage_armed = false;

inline void mark(void* const* ev, int i, hipStream_t s)
{
    if (ev != nullptr && ev[i] != nullptr)
        (void)hipEventRecord((hipEvent_t)ev[i], s);
}

// largest K the skinny GEMM stages per-row side data for (LDS budget 48 KB),
// with `group` K per activation scale
bool skinny_k_ok(int64_t K, int block_m, int64_t group = W4A8_GROUP)
{
    return (K / group) * block_m * 8 <= 48 * 1024;
}

}  // namespace

extern "C" {

int w4a8_version(void)
{
    return (0 << 16) | 1;
}

const char* w4a8_status_string(int status)
{
    switch (status) {
    case W4A8_OK: return "ok";
    case W4A8_ERR_INVALID_ARG: return "invalid argument";
    case W4A8_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case W4A8_ERR_WORKSPACE: return "workspace too small";
    case W4A8_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

int w4a8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, uint8_t* q_e4m3,
                      float* scales, hipStream_t stream)
{
    if (M < 0 || K <= 0 || ldx < K)
        return W4A8_ERR_INVALID_ARG;
    if (M > 0 && (x_bf16 == nullptr || q_e4m3 == nullptr || scales == nullptr))
        return W4A8_ERR_INVALID_ARG;
    if (K % W4A8_GROUP != 0 || ldx % 8 != 0)
        return W4A8_ERR_UNSUPPORTED;
    // one workgroup per 16 blocks of 128: the grid stays within 2^31 - 1
    if (ceil_div(mul_sat(M, K / W4A8_GROUP), 16) > INT32_MAX)
        return W4A8_ERR_UNSUPPORTED;
    if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(scales))
        return W4A8_ERR_UNSUPPORTED;
    if (M == 0)
        return W4A8_OK;
    return hip_status(w4a8::launch_quant_bf16((const uint16_t*)x_bf16, M, K, ldx, q_e4m3, scales,
                                              nullptr, 0, nullptr, stream));
}

int w4a8_gemm(const uint8_t* a_e4m3, const float* a_scales, int64_t M, int64_t K,
              const uint8_t* b_int4, const float* b_scales, int64_t N, void* out_bf16,
              void* workspace, size_t* workspace_bytes, hipStream_t stream)
{
    if (M < 0 || K <= 0 || N <= 0)
        return W4A8_ERR_INVALID_ARG;
    if (K % W4A8_GROUP != 0)
        return W4A8_ERR_UNSUPPORTED;
    // 32-bit buffer ranges: the activation codes [M, K] and the weights [N, K/2];
    // 128-row blocks on grid.y
    if (!below_u32(mul_sat(M, K)) || !below_u32(mul_sat(N, K / 2)) || ceil_div(M, 128) > kMaxGridY)
        return W4A8_ERR_UNSUPPORTED;
    float* part;
    const size_t need = plan_gemm(nullptr, M, K, N, &part);
    const int ws_rc = check_workspace(workspace, workspace_bytes, need);
    if (ws_rc >= 0)
        return ws_rc;
    if (M > 0 && (a_e4m3 == nullptr || a_scales == nullptr || out_bf16 == nullptr))
        return W4A8_ERR_INVALID_ARG;
    if (b_int4 == nullptr || b_scales == nullptr)
        return W4A8_ERR_INVALID_ARG;
    if (!aligned16(a_e4m3) || !aligned16(b_int4) || !aligned16(out_bf16) ||
        !aligned16(a_scales) || !aligned16(b_scales))
        return W4A8_ERR_UNSUPPORTED;
    if (M == 0)
        return W4A8_OK;
    plan_gemm(workspace, M, K, N, &part);
    const int32_t gps = gemm_split_groups(M, K, N);
    hipError_t e = w4a8::launch_dense_gemm(a_e4m3, a_scales, M, K, b_int4, b_scales, N, gps, part,
                                           (uint16_t*)out_bf16, stream);
    if (e != hipSuccess || part == nullptr)
        return hip_status(e);
    // the slices' partial sums, in slice order, one bf16 rounding
    return hip_status(w4a8::launch_split_reduce(part, (int32_t)ceil_div(K / W4A8_GROUP, gps), M, N,
                                                (uint16_t*)out_bf16, stream));
}

int w4a8_moe_align(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t expert_begin,
                   int64_t num_local_experts, int64_t block_m, int32_t* expert_counts,
                   int32_t* expert_offsets, int32_t* sorted_pair_ids, int32_t* src2dst,
                   int32_t* block_expert, int32_t* block_row, int32_t* num_blocks,
                   void* workspace, size_t* workspace_bytes, hipStream_t stream)
{
    if (T < 0 || topk < 1 || num_local_experts < 1 || block_m < 1)
        return W4A8_ERR_INVALID_ARG;
    if (topk > W4A8_MAX_TOPK || num_local_experts > kMaxLocalExperts || mul_sat(T, topk) > INT32_MAX / 2)
        return W4A8_ERR_UNSUPPORTED;
    const size_t need = round_up(w4a8::align_workspace_bytes(T * topk, num_local_experts));
    const int ws_rc = check_workspace(workspace, workspace_bytes, need);
    if (ws_rc >= 0)
        return ws_rc;
    if ((T > 0 && (topk_ids == nullptr || sorted_pair_ids == nullptr || src2dst == nullptr)) ||
        expert_counts == nullptr || expert_offsets == nullptr || num_blocks == nullptr ||
        ((block_expert == nullptr) != (block_row == nullptr)))
        return W4A8_ERR_INVALID_ARG;
    w4a8::AlignOut o = {expert_counts, expert_offsets, sorted_pair_ids, src2dst,
                        block_expert, block_row, num_blocks, nullptr};
    return hip_status(w4a8::launch_align(topk_ids, T, topk, expert_begin, num_local_experts,
                                         block_m, o, workspace, stream));
}

}  // extern "C"

namespace {

// weight formats of the fused forward
enum WeightFormat { kInt4 = 0, kInt4Packed = 1, kFp4Packed = 2 };

// the same GEMM's arguments for the second m-block list (32-row blocks)
w4a8::GemmArgs second_list(const w4a8::GemmArgs& g, const MoePlan& p)
{
    w4a8::GemmArgs g2 = g;
    g2.block_expert = p.al.block_expert2;
    g2.block_row = p.al.block_row2;
    g2.num_blocks = p.al.num_blocks2;
    g2.max_blocks = p.nb2_max;
    return g2;
}

// the same GEMM's arguments for the block-tiled list of a device-chosen path
w4a8::GemmArgs tiled_list(const w4a8::GemmArgs& g, const MoePlan& p)
{
    w4a8::GemmArgs g3 = g;
    g3.block_expert = nullptr;
    g3.block_row = p.al.block_row3;
    g3.num_blocks = p.al.num_blocks3;
    g3.max_blocks = p.nb3_max;
    g3.path = p.al.path;
    g3.path_want = 1;
    return g3;
}

// one GEMM stage on the plan's path(s): the block-tiled kernel, the skinny
// kernel over one or two lists, or (device-chosen) both, one of which exits
hipError_t launch_stage(const w4a8::GemmArgs& g, const MoePlan& p, bool gate_up, hipStream_t s)
{
    const int tile_mode = gate_up ? w4a8::TILE_GATEUP : w4a8::TILE_DOWN;
    const int epi = gate_up ? w4a8::EPI_SWIGLU_Q : w4a8::EPI_F32;
    if (p.tile)
        return w4a8::launch_gemm_tile(g, tile_mode, s);
    if (!p.two_lists)
        return w4a8::launch_gemm_skinny(g, epi, p.block_m, s);
    if (p.choose) {
        const hipError_t e = w4a8::launch_gemm_tile(tiled_list(g, p), tile_mode, s);
        if (e != hipSuccess)
            return e;
        w4a8::GemmArgs g1 = g;
        g1.path = p.al.path;
        g1.path_want = 0;
        return w4a8::launch_gemm_skinny_two_lists(g1, second_list(g1, p), epi, s);
    }
    return w4a8::launch_gemm_skinny_two_lists(g, second_list(g, p), epi, s);
}

// ev: the stage events to record (null: none); max_pairs, pairs_out: the
// bound on the local pairs and where their count goes (0 / null: none)
int fused_moe_run(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                  const float* topk_weights, int64_t topk, int64_t expert_begin,
                  int64_t num_local_experts, int64_t I, const uint8_t* w13_int4,
                  const void* w13_scales, const uint8_t* w2_int4, const void* w2_scales,
                  void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream,
                  WeightFormat format, const float* a1_scale, const float* a2_scale, int down_group,
                  void* const* ev, int64_t max_pairs = 0, int32_t* pairs_out = nullptr,
                  bool persistent = false)
{
    const bool packed = format != kInt4;
    if (down_group != 128 && down_group != 64 && down_group != 32)
        return W4A8_ERR_INVALID_ARG;
    if (down_group != W4A8_GROUP && !packed)
        return W4A8_ERR_UNSUPPORTED;  // the finer recipes read prepacked weights
    const int64_t E = num_local_experts;
    if (T < 0 || H <= 0 || I <= 0 || topk < 1 || E < 1)
        return W4A8_ERR_INVALID_ARG;
    if (H % W4A8_GROUP != 0 || I % W4A8_GROUP != 0 || topk > W4A8_MAX_TOPK ||
        E > kMaxLocalExperts || mul_sat(T, topk) > INT32_MAX / 2)
        return W4A8_ERR_UNSUPPORTED;
    MoePlan p;
    const size_t need = plan_moe(nullptr, T, H, topk, E, I, p, down_group, max_pairs, persistent);
    // 32-bit buffer ranges: the gate_up operand [T, H], the down operand
    // [cap, I] (cap = T*topk unless bounded), one expert's w13 [2I, H/2]
    if (!below_u32(mul_sat(T, H)) || !below_u32(mul_sat(p.cap, I)) || !below_u32(mul_sat(I, H)))
        return W4A8_ERR_UNSUPPORTED;
    // the single-launch combine counts (token, 8-column) items of a block of
    // 64 tokens in 32 bits
    if (persistent && H > kMaxPersistentH)
        return W4A8_ERR_UNSUPPORTED;
    if (!p.tile && (!skinny_k_ok(H, p.block_m) || !skinny_k_ok(I, p.block_m, down_group) ||
                    p.nb_max > kMaxGridY ||
                    (p.two_lists && (!skinny_k_ok(H, kLargeBlockRows) || !skinny_k_ok(I, kLargeBlockRows) ||
                                     p.nb_max + p.nb2_max > kMaxGridY))))
        return W4A8_ERR_UNSUPPORTED;
    const int ws_rc = check_workspace(workspace, workspace_bytes, need);
    if (ws_rc >= 0)
        return ws_rc;
    if (T > 0 && (hidden_bf16 == nullptr || topk_ids == nullptr || topk_weights == nullptr ||
                  out_bf16 == nullptr))
        return W4A8_ERR_INVALID_ARG;
    if (w13_int4 == nullptr || w13_scales == nullptr || w2_int4 == nullptr || w2_scales == nullptr)
        return W4A8_ERR_INVALID_ARG;
    if (!aligned16(hidden_bf16) || !aligned16(out_bf16) || !aligned16(w13_int4) ||
        !aligned16(w2_int4) || !aligned16(w13_scales) || !aligned16(w2_scales))
        return W4A8_ERR_UNSUPPORTED;
    if (T == 0)
        return W4A8_OK;
    plan_moe(workspace, T, H, topk, E, I, p, down_group, max_pairs, persistent);
    p.al.pairs_out = pairs_out;

    mark(ev, 0, stream);
    hipError_t e;
    if (w4a8::align_chunk_count(p.F) == 1) {
        // few pairs: align and quantisation in one launch (both stage events
        // are recorded after it)
        e = w4a8::launch_align_quant(topk_ids, T, topk, expert_begin, E, p.block_m, p.al,
                                     (const uint16_t*)hidden_bf16, H, p.qa, p.qa_side, a1_scale,
                                     stream);
        if (e != hipSuccess)
            return W4A8_ERR_HIP;
        mark(ev, 1, stream);
    } else {
        // many pairs: the quantisation's blocks ride along with the align's
        // count and scatter launches (both stage events after them)
        const w4a8::QuantJob qj = {(const uint16_t*)hidden_bf16, T, H, H, p.qa, p.qa_side, a1_scale};
        e = w4a8::launch_align(topk_ids, T, topk, expert_begin, E, p.block_m, p.al, p.align_ws,
                               stream, qj);
        if (e != hipSuccess)
            return W4A8_ERR_HIP;
        mark(ev, 1, stream);
    }
    mark(ev, 2, stream);

    w4a8::GemmArgs g = {};
    g.sub_group = W4A8_GROUP;
    g.block_expert = p.al.block_expert;
    g.block_row = p.al.block_row;
    g.num_blocks = p.al.num_blocks;
    g.offsets = p.al.offsets;
    g.block_start = p.block_start;
    g.num_experts = (int32_t)E;
    g.max_blocks = p.nb_max;
    // gate_up: rows gathered through the permutation, exact f16 MFMA path,
    // SwiGLU + requant epilogue
    g.act = p.qa;
    g.act_rows = T;
    g.f16 = 1;
    g.act_side = p.qa_side;
    g.sorted = p.al.sorted;
    g.topk = (int32_t)topk;
    g.packed = packed ? 1 : 0;
    g.fp4 = format == kFp4Packed ? 1 : 0;
    g.w = w13_int4;
    g.ws = (const float*)w13_scales;
    g.w_estride = 2 * I * (H / 2);
    g.s_estride = 2 * I * (packed ? 4 * ceil_div(H / W4A8_GROUP, 4) : H / W4A8_GROUP);
    g.K = H;
    g.N = 2 * I;
    g.I = I;
    g.out_q = p.qh;
    g.out_side = p.qh_side;
    g.requant_scale = a2_scale;
    g.sub_group = down_group;
    const w4a8::GemmArgs gu = g;
    if (!persistent) {
        e = launch_stage(g, p, true, stream);
        if (e != hipSuccess)
            return W4A8_ERR_HIP;
        mark(ev, 3, stream);
    }
    // down: rows in pair order, fp8 MFMA path
    g.act = p.qh;
    g.act_rows = p.cap;
    g.f16 = 0;
    g.act_side = p.qh_side;
    g.sorted = nullptr;
    g.w = w2_int4;
    g.ws = (const float*)w2_scales;
    g.w_estride = H * (I / 2);
    g.s_estride = H * (packed ? 4 * ceil_div(I / W4A8_GROUP, 4) : I / W4A8_GROUP);
    g.K = I;
    g.N = H;
    g.out_f32 = p.y2;
    if (persistent) {
        // gate_up, down and combine in one launch (the stage events after it)
        const w4a8::TailArgs tail = {p.y2, p.al.src2dst, topk_weights, T, topk, H,
                                     (uint16_t*)out_bf16, p.al.barrier};
        e = w4a8::launch_fused_tail(gu, g, tail, stream);
        if (e != hipSuccess)
            return W4A8_ERR_HIP;
        mark(ev, 3, stream);
        mark(ev, 4, stream);
        mark(ev, 5, stream);
        return W4A8_OK;
    }
    e = launch_stage(g, p, false, stream);
    if (e != hipSuccess)
        return W4A8_ERR_HIP;
    mark(ev, 4, stream);
    e = w4a8::launch_combine(p.y2, p.al.src2dst, topk_weights, T, topk, H, (uint16_t*)out_bf16,
                             stream);
    if (e != hipSuccess)
        return W4A8_ERR_HIP;
    mark(ev, 5, stream);
    return W4A8_OK;
}

// any call of the family consumes the stage-event arming (see the header)
void* const* take_stage_events()
{
    const bool timed = t_stage_armed;
    t_stage_armed = false;
    return timed ? t_stage_events : nullptr;
}

int fused_moe_impl(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                   const float* topk_weights, int64_t topk, int64_t expert_begin,
                   int64_t num_local_experts, int64_t I, const uint8_t* w13_int4,
                   const void* w13_scales, const uint8_t* w2_int4, const void* w2_scales,
                   void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream,
                   WeightFormat format, const float* a1_scale = nullptr,
                   const float* a2_scale = nullptr, int down_group = W4A8_GROUP,
                   int64_t max_pairs = 0, int32_t* pairs_out = nullptr, bool persistent = false)
{
    void* const* ev = take_stage_events();
    return fused_moe_run(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                         num_local_experts, I, w13_int4, w13_scales, w2_int4, w2_scales, out_bf16,
                         workspace, workspace_bytes, stream, format, a1_scale, a2_scale, down_group, ev,
                         max_pairs, pairs_out, persistent);
}

}  // namespace

extern "C" {

int w4a8_fused_moe(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                   const float* topk_weights, int64_t topk, int64_t expert_begin,
                   int64_t num_local_experts, int64_t I, const uint8_t* w13_int4,
                   const float* w13_scales, const uint8_t* w2_int4, const float* w2_scales,
                   void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream)
{
    return fused_moe_impl(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13_int4, w13_scales, w2_int4, w2_scales, out_bf16,
                          workspace, workspace_bytes, stream, kInt4);
}

int w4a8_fused_moe_prepacked(const void* hidden_bf16, int64_t T, int64_t H,
                             const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                             int64_t expert_begin, int64_t num_local_experts, int64_t I,
                             const uint8_t* w13_packed, const float* w13_scales_packed,
                             const uint8_t* w2_packed, const float* w2_scales_packed,
                             void* out_bf16, void* workspace, size_t* workspace_bytes,
                             hipStream_t stream)
{
    return fused_moe_impl(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13_packed, w13_scales_packed, w2_packed,
                          w2_scales_packed, out_bf16, workspace, workspace_bytes, stream, kInt4Packed);
}

int w4a8_fused_moe_prepacked_static(const void* hidden_bf16, int64_t T, int64_t H,
                                    const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                                    int64_t expert_begin, int64_t num_local_experts, int64_t I,
                                    const uint8_t* w13_packed, const float* w13_scales_packed,
                                    const uint8_t* w2_packed, const float* w2_scales_packed,
                                    const float* a1_scale, const float* a2_scale, void* out_bf16,
                                    void* workspace, size_t* workspace_bytes, hipStream_t stream)
{
    if (((uintptr_t)a1_scale & 3u) != 0 || ((uintptr_t)a2_scale & 3u) != 0) {
        (void)take_stage_events();  // a rejected call disarms the stage events too
        return W4A8_ERR_UNSUPPORTED;
    }
    return fused_moe_impl(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13_packed, w13_scales_packed, w2_packed,
                          w2_scales_packed, out_bf16, workspace, workspace_bytes, stream, kInt4Packed,
                          a1_scale, a2_scale);
}

int w4a8_fused_moe_recipe(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                          const float* topk_weights, int64_t topk, int64_t expert_begin,
                          int64_t num_local_experts, int64_t I, int weight_format,
                          const uint8_t* w13_packed, const void* w13_scales_packed,
                          const uint8_t* w2_packed, const void* w2_scales_packed, int down_act_group,
                          void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream)
{
    if (weight_format != W4A8_WEIGHTS_INT4_PACKED && weight_format != W4A8_WEIGHTS_FP4_PACKED) {
        (void)take_stage_events();  // a rejected call disarms the stage events too
        return W4A8_ERR_INVALID_ARG;
    }
    return fused_moe_impl(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13_packed, w13_scales_packed, w2_packed,
                          w2_scales_packed, out_bf16, workspace, workspace_bytes, stream,
                          weight_format == W4A8_WEIGHTS_FP4_PACKED ? kFp4Packed : kInt4Packed,
                          nullptr, nullptr, down_act_group);
}

int w4a8_fused_moe_fp4_prepacked(const void* hidden_bf16, int64_t T, int64_t H,
                                 const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                                 int64_t expert_begin, int64_t num_local_experts, int64_t I,
                                 const uint8_t* w13_packed, const uint32_t* w13_scales_packed,
                                 const uint8_t* w2_packed, const uint32_t* w2_scales_packed,
                                 void* out_bf16, void* workspace, size_t* workspace_bytes,
                                 hipStream_t stream)
{
    return fused_moe_impl(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                          num_local_experts, I, w13_packed, w13_scales_packed, w2_packed,
                          w2_scales_packed, out_bf16, workspace, workspace_bytes, stream, kFp4Packed);
}

int w4a8_fused_moe_bounded(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                           const float* topk_weights, int64_t topk, int64_t expert_begin,
                           int64_t num_local_experts, int64_t I, int weight_format,
                           const uint8_t* w13, const void* w13_scales, const uint8_t* w2,
                           const void* w2_scales, int64_t max_local_pairs, int32_t* local_pairs,
                           void* out_bf16, void* workspace, size_t* workspace_bytes, hipStream_t stream)
{
    void* const* ev = take_stage_events();  // consumed by rejected calls too
    if (weight_format != W4A8_WEIGHTS_INT4 && weight_format != W4A8_WEIGHTS_INT4_PACKED &&
        weight_format != W4A8_WEIGHTS_FP4_PACKED)
        return W4A8_ERR_INVALID_ARG;
    if (max_local_pairs < 1 || (workspace != nullptr && T > 0 && local_pairs == nullptr))
        return W4A8_ERR_INVALID_ARG;
    if (((uintptr_t)local_pairs & 7u) != 0)
        return W4A8_ERR_UNSUPPORTED;
    const WeightFormat f = weight_format == W4A8_WEIGHTS_FP4_PACKED    ? kFp4Packed
                           : weight_format == W4A8_WEIGHTS_INT4_PACKED ? kInt4Packed
                                                                       : kInt4;
    return fused_moe_run(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                         num_local_experts, I, w13, w13_scales, w2, w2_scales, out_bf16, workspace,
                         workspace_bytes, stream, f, nullptr, nullptr, W4A8_GROUP, ev, max_local_pairs,
                         local_pairs);
}

int w4a8_fused_moe_persistent(const void* hidden_bf16, int64_t T, int64_t H, const int32_t* topk_ids,
                              const float* topk_weights, int64_t topk, int64_t expert_begin,
                              int64_t num_local_experts, int64_t I, int weight_format,
                              const uint8_t* w13, const void* w13_scales, const uint8_t* w2,
                              const void* w2_scales, void* out_bf16, void* workspace,
                              size_t* workspace_bytes, hipStream_t stream)
{
    void* const* ev = take_stage_events();  // consumed by rejected calls too
    if (weight_format != W4A8_WEIGHTS_INT4 && weight_format != W4A8_WEIGHTS_INT4_PACKED &&
        weight_format != W4A8_WEIGHTS_FP4_PACKED)
        return W4A8_ERR_INVALID_ARG;
    const WeightFormat f = weight_format == W4A8_WEIGHTS_FP4_PACKED    ? kFp4Packed
                           : weight_format == W4A8_WEIGHTS_INT4_PACKED ? kInt4Packed
                                                                       : kInt4;
    return fused_moe_run(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                         num_local_experts, I, w13, w13_scales, w2, w2_scales, out_bf16, workspace,
                         workspace_bytes, stream, f, nullptr, nullptr, W4A8_GROUP, ev, 0, nullptr,
                         true);
}

int w4a8_prepack_weights(const uint8_t* w_int4, const float* w_scales, int64_t E, int64_t N,
                         int64_t K, uint8_t* w_packed, float* s_packed, hipStream_t stream)
{
    if (E < 1 || N <= 0 || K <= 0)
        return W4A8_ERR_INVALID_ARG;
    if (w_int4 == nullptr || w_scales == nullptr || w_packed == nullptr || s_packed == nullptr)
        return W4A8_ERR_INVALID_ARG;
    if (N % 16 != 0 || K % W4A8_GROUP != 0)
        return W4A8_ERR_UNSUPPORTED;
    // one expert's weights stay below 2^32 bytes (the GEMMs' buffer ranges);
    // one thread per 16 bytes: the grid stays within 2^31 - 1 workgroups
    if (!below_u32(mul_sat(N, K / 2)) || ceil_div(mul_sat(E, N * (K / 2)), 16 * 256) > INT32_MAX)
        return W4A8_ERR_UNSUPPORTED;
    if (!aligned16(w_int4) || !aligned16(w_packed) || !aligned16(w_scales) || !aligned16(s_packed))
        return W4A8_ERR_UNSUPPORTED;
    if ((const void*)w_int4 == (const void*)w_packed || (const void*)w_scales == (const void*)s_packed)
        return W4A8_ERR_INVALID_ARG;  // not in place
    return hip_status(w4a8::launch_prepack(w_int4, w_scales, E, N, K, false, false, w_packed, s_packed,
                                           stream));
}

int w4a8_prepack_weights_bf16_scales(const uint8_t* w_int4, const uint16_t* w_scales_bf16, int64_t E,
                                     int64_t N, int64_t K, uint8_t* w_packed, float* s_packed,
                                     hipStream_t stream)
{
    if (E < 1 || N <= 0 || K <= 0)
        return W4A8_ERR_INVALID_ARG;
    if (w_int4 == nullptr || w_scales_bf16 == nullptr || w_packed == nullptr || s_packed == nullptr)
        return W4A8_ERR_INVALID_ARG;
    if (N % 16 != 0 || K % W4A8_GROUP != 0)
        return W4A8_ERR_UNSUPPORTED;
    // one expert's weights stay below 2^32 bytes (the GEMMs' buffer ranges);
    // one thread per 16 bytes: the grid stays within 2^31 - 1 workgroups
    if (!below_u32(mul_sat(N, K / 2)) || ceil_div(mul_sat(E, N * (K / 2)), 16 * 256) > INT32_MAX)
        return W4A8_ERR_UNSUPPORTED;
    if (!aligned16(w_int4) || !aligned16(w_packed) || ((uintptr_t)w_scales_bf16 & 1u) != 0 ||
        !aligned16(s_packed))
        return W4A8_ERR_UNSUPPORTED;
    if ((const void*)w_int4 == (const void*)w_packed ||
        (const void*)w_scales_bf16 == (const void*)s_packed)
        return W4A8_ERR_INVALID_ARG;  // not in place
    return hip_status(w4a8::launch_prepack(w_int4, w_scales_bf16, E, N, K, false, true, w_packed,
                                           s_packed, stream));
}

int w4a8_prepack_weights_fp4(const uint8_t* w_fp4, const uint8_t* w_scales_ue8m0, int64_t E,
                             int64_t N, int64_t K, int role, uint8_t* w_packed,
                             uint32_t* s_packed, hipStream_t stream)
{
    if (E < 1 || N <= 0 || K <= 0)
        return W4A8_ERR_INVALID_ARG;
    if (role != W4A8_FP4_GATE_UP && role != W4A8_FP4_DOWN)
        return W4A8_ERR_INVALID_ARG;
    if (w_fp4 == nullptr || w_scales_ue8m0 == nullptr || w_packed == nullptr || s_packed == nullptr)
        return W4A8_ERR_INVALID_ARG;
    if (N % 16 != 0 || K % W4A8_GROUP != 0)
        return W4A8_ERR_UNSUPPORTED;
    // one expert's weights stay below 2^32 bytes (the GEMMs' buffer ranges);
    // one thread per 16 bytes: the grid stays within 2^31 - 1 workgroups
    if (!below_u32(mul_sat(N, K / 2)) || ceil_div(mul_sat(E, N * (K / 2)), 16 * 256) > INT32_MAX)
        return W4A8_ERR_UNSUPPORTED;
    // the scales are moved as one dword per row and 128-group
    if (!aligned16(w_fp4) || !aligned16(w_packed) || ((uintptr_t)w_scales_ue8m0 & 3u) != 0 ||
        !aligned16(s_packed))
        return W4A8_ERR_UNSUPPORTED;
    if ((const void*)w_fp4 == (const void*)w_packed ||
        (const void*)w_scales_ue8m0 == (const void*)s_packed)
        return W4A8_ERR_INVALID_ARG;  // not in place
    return hip_status(w4a8::launch_prepack(w_fp4, w_scales_ue8m0, E, N, K, role == W4A8_FP4_GATE_UP,
                                           false, w_packed, s_packed, stream));
}

int64_t w4a8_prepacked_scale_count(int64_t E, int64_t N, int64_t K)
{
    if (E < 1 || N <= 0 || K <= 0 || K % W4A8_GROUP != 0)
        return -1;
    return E * N * 4 * ceil_div(K / W4A8_GROUP, 4);
}

int w4a8_fused_moe_workspace_layout(int64_t T, int64_t H, int64_t topk,
                                    int64_t num_local_experts, int64_t I, size_t* offsets, int n,
                                    int64_t* block_m)
{
    if (T < 0 || H <= 0 || I <= 0 || topk < 1 || num_local_experts < 1 || offsets == nullptr ||
        (n != 12 && n != 15 && n != 18) || block_m == nullptr)
        return W4A8_ERR_INVALID_ARG;
    MoePlan p;
    // carve from a fake base so that pointers equal byte offsets (base != null)
    char* const base = (char*)(uintptr_t)4096;
    plan_moe(base, T, H, topk, num_local_experts, I, p);
    const void* ptrs[18] = {p.al.counts, p.al.offsets, p.al.sorted, p.al.src2dst,
                            p.al.block_expert, p.al.block_row, p.al.num_blocks, p.qa,
                            p.qa_side, p.qh, p.qh_side, p.y2,
                            p.al.block_expert2, p.al.block_row2, p.al.num_blocks2,
                            p.al.block_row3, p.al.num_blocks3, p.al.path};
    for (int i = 0; i < n; ++i)
        offsets[i] = ptrs[i] != nullptr ? (size_t)((const char*)ptrs[i] - base) : 0;
    *block_m = p.block_m;
    return W4A8_OK;
}

int w4a8_fused_moe_stage_events(void* const* events, int n)
{
    if (n == 0) {
        t_stage_armed = false;
        return W4A8_OK;
    }
    if (n != 6 || events == nullptr)
        return W4A8_ERR_INVALID_ARG;
    for (int i = 0; i < 6; ++i)
        t_stage_events[i] = events[i];
    t_stage_armed = true;
    return W4A8_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free fused forward: the workspace is a file-scope device array.
// Each GPU the library runs on holds its own copy until the process ends.
// The host never passes the array's name to a kernel: the address comes from
// hipGetSymbolAddress, once per device with that device current.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) uint8_t scratch[W4A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of the current device's scratch array (null on failure)
void* scratch_of_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int w4a8_fused_moe_prepacked_noalloc(const void* hidden_bf16, int64_t T, int64_t H,
                                     const int32_t* topk_ids, const float* topk_weights, int64_t topk,
                                     int64_t expert_begin, int64_t num_local_experts, int64_t I,
                                     const uint8_t* w13_packed, const float* w13_scales_packed,
                                     const uint8_t* w2_packed, const float* w2_scales_packed,
                                     void* out_bf16, hipStream_t stream)
{
    void* const* ev = take_stage_events();
    // the workspace this call needs (host-only query, validates the shapes)
    size_t need = 0;
    const int q = fused_moe_run(nullptr, T, H, nullptr, nullptr, topk, expert_begin,
                                num_local_experts, I, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, &need, stream, kInt4Packed, nullptr, nullptr, W4A8_GROUP,
                                nullptr);
    if (q != W4A8_OK)
        return q;
    if (need > (size_t)W4A8_NOALLOC_SCRATCH_BYTES)
        return W4A8_ERR_WORKSPACE;
    void* ws = scratch_of_current_device();
    if (ws == nullptr)
        return W4A8_ERR_HIP;
    size_t bytes = (size_t)W4A8_NOALLOC_SCRATCH_BYTES;
    return fused_moe_run(hidden_bf16, T, H, topk_ids, topk_weights, topk, expert_begin,
                         num_local_experts, I, w13_packed, w13_scales_packed, w2_packed,
                         w2_scales_packed, out_bf16, ws, &bytes, stream, kInt4Packed, nullptr, nullptr,
                         W4A8_GROUP, ev);
}

}  // extern "C"
