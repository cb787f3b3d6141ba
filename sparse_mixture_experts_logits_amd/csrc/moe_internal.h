// Internal declarations shared by the HIP translation units of the MoE
// library: device helpers, workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ device helpers

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

struct alignas(16) u32x4 {
    uint32_t x, y, z, w;
};

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// Plain 16-byte load (one dwordx4 instruction).
__device__ __forceinline__ u32x4 load16(const void *p)
{
    const u32x4v_t v = *reinterpret_cast<const u32x4v_t *>(p);
    return u32x4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + (((u >> 16) & 1u) + 0x7fffu)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// ------------------------------------------------------------------ routing constants

constexpr int kRouterMaxTokensPerBlock = 4;  // tokens per router block: 1 or 4
constexpr int kMaxExperts = 256;

// Device tile of the large-M grouped GEMM: rows [row0, row0 + rows) of the
// expert-sorted assignment list, all belonging to expert `expert`.
struct alignas(16) MTile {
    int32_t expert;
    int32_t row0;
    int32_t rows;
    int32_t pad;
};

// ------------------------------------------------------------------ workspace

struct Workspace {
    int32_t *ids;          // [TK] selected experts, flat t*k+j
    float *wts;            // [TK] routed weights (x routed_scale)
    int32_t *blk_counts;   // [nblk][E] per-router-block histogram
    int32_t *blk_base;     // [nblk][E] first sorted position of each block's run
    float *blk_prob;       // [nblk][E] router-probability sums of the block's counted tokens
    int32_t *blk_mcnt;     // [nblk][E] assignments of the block's counted tokens
    int32_t *blk_ntok;     // [nblk] counted tokens of the block
    int32_t *counts;       // [E]
    int32_t *offsets;      // [E+1]
    int32_t *tile_start;   // [E+1] first M-tile of each expert (large-M schedule)
    MTile *tiles;          // [max_tiles]
    int32_t *perm;         // [TK] sorted position -> flat assignment
    int32_t *inv;          // [TK] flat assignment -> sorted position
    int32_t *row_token;    // [TK] sorted position -> token
    float *row_weight;     // [TK] sorted position -> routed weight
    int32_t *row_expert;   // [TK] sorted position -> expert
    void *h;               // [TK, I] activation of the routed experts (bf16 or f32)
    float *slot;           // [TK, H] weighted routed outputs, flat-assignment order
    void *sh_h;            // [T, shared_I] shared-expert activation
    float *sh_y;           // [T, H] shared-expert output
    float *part;           // large-M schedule: partial sums of split tiles (or null)
};

// Tile blocks (MOE_LAYOUT_TILE_BLOCKS): 256 weight rows x 32 columns per block.
constexpr int kBlockRows = 256;
constexpr int kBlockCols = 32;

struct Shape {
    int64_t T, H, I, E;
    int k;
    int64_t sharedI;
    int dtype;       // 0 bf16, 1 f32
    int rtok;        // tokens per router block (1 or 4)
    int nblk;        // router blocks
    int tileBM;      // rows per M-tile of the large-M schedule
    int tileXT;      // extra rows an expert's last M-tile may take (0: none)
    int tileMinRows; // experts with fewer rows get no M-tile (mixed schedule; 0: every expert)
    int64_t maxTiles;
    int64_t partBytes;  // partial-sum buffer (0 unless the large-M schedule may run)
    bool hBlocks;       // h in row blocks of the tile list (bf16 tiled schedule, see below)
};

// h in row blocks (bf16, tiled schedule only): gate_up's tile i writes its
// rows as [i][kt][kHBlockRows][kBlockCols], one contiguous 18 KB run per
// 32-column stage, so that every copy of the down GEMM's token rows reads
// 1 KB contiguous. Rows past the tile's own and columns past I are never
// written (the down copies clamp the rows and mask the columns).
constexpr int kHBlockRows = 288;  // rows of an M-tile with its extra rows
inline int64_t h_blocks_bytes(int64_t tiles, int64_t I)
{
    return tiles * ((I + kBlockCols - 1) / kBlockCols) * kHBlockRows * kBlockCols * 2;
}

// Byte layout of the workspace; returns total bytes, fills ws when base != null.
int64_t workspace_layout(const Shape &s, void *base, Workspace *ws);

// ------------------------------------------------------------------ launchers (return hipError_t)

// Optional router statistics (load-balancing loss inputs).
struct RouterStats {
    const int32_t *mask;  // [T] nonzero = counted; null = every token
    float *prob_mean;     // [E]
    float *load;          // [E]
    float *aux;           // [1]
    bool on() const { return prob_mean || load || aux; }
};

// Scoring variant of the router (softmax by default).
constexpr int kMaxGroups = 64;
struct RouterCfg {
    int score_func = 0;               // 0 softmax, 1 sigmoid, 2 sparsemixer
    const float *sel_bias = nullptr;  // [E] added to selection keys only
    int n_group = 0;                  // > 1: group-limited selection
    int topk_group = 0;
    float jitter_eps = 0.0f;          // sparsemixer threshold
};

hipError_t launch_router_topk(const Shape &s, const void *X, const void *Wr, const float *bias,
                              float routed_scale, float *logits_out, int32_t *ids_out, float *wts_out,
                              const RouterStats &rs, const RouterCfg &rc, const Workspace &ws, hipStream_t st);
hipError_t launch_route_scan(const Shape &s, int32_t *counts_out, int32_t *offsets_out,
                             const RouterStats &rs, const Workspace &ws, hipStream_t st);
hipError_t launch_route_permute(const Shape &s, int32_t *perm_out, int32_t *inv_out,
                                const Workspace &ws, hipStream_t st);

// Grouped expert GEMMs. `dense_rows` > 0 selects the dense form used by the
// shared expert: one group, rows [0, dense_rows), identity row maps.
struct GemmProblem {
    const void *A;           // gate_up: hidden [T, K]; down: h [rows, K]
    const int32_t *a_rows;   // gate_up: sorted position -> token (null = identity)
    const void *W;           // packed weights (bf16 / fp32, or E4M3 bytes when w_scale is set)
    const float *w_scale;    // E4M3 storage: per-row scales [E, rows per expert]; else null
    const uint8_t *w_bscale = nullptr;  // MXFP4 storage: E8M0 block scales [E, rows, K / 32]; else null
    int64_t w_expert_stride; // elements between experts (0 for dense)
    int64_t K;               // reduction length
    int64_t N;               // gate_up: I (h columns); down: H
    void *C;                 // gate_up: h [rows, N]; down: fp32 [.., N]
    const int32_t *c_rows;   // down: sorted position -> output row (null = identity)
    const float *c_scale;    // down: sorted position -> weight (null = 1)
    const int32_t *counts;   // [E] rows per expert (null in dense form)
    const int32_t *offsets;  // [E+1]
    const int32_t *row_expert;  // [rows] (fp32 path)
    const MTile *tiles;      // large-M schedule
    const int32_t *tile_start;  // [E+1]
    int64_t E;
    int64_t dense_rows;
    int64_t total_rows;      // host-known number of rows (TK or T)
    float *part = nullptr;   // large-M schedule: partial sums of split tiles (null: no splitting)
    // weight-streaming schedule, direct routing: rows taken straight from the
    // top-k ids (no sorted tables; see the skinny kernel)
    const int32_t *ids = nullptr;
    const float *wts = nullptr;
    int k = 0;
    int cus = 0;             // compute units of the device (persistent grids)
    int64_t a_rows_total = 0;  // rows of A (gate_up: tokens; down: assignments or tokens)
    int skinny_max_rows = 0;   // > 0: the weight-streaming launch leaves experts with more rows to the tiled one
    bool w_blocks = false;     // routed weights in tile blocks (MOE_LAYOUT_TILE_BLOCKS; tiled kernels only)
    bool h_blocks = false;     // tiled routed launches: gate_up writes C, down reads A, as h row blocks
    int64_t h_bytes = 0;       // bytes of the h row blocks (their buffer resource bound)
};

// Bytes of one expert's tile blocks (which: MOE_PACK_GATE_UP / MOE_PACK_DOWN).
inline int64_t tile_blocks_expert_bytes(int which, int64_t I, int64_t H)
{
    const int64_t nb = which == 0 ? (I + 127) / 128 : (H + kBlockRows - 1) / kBlockRows;
    const int64_t nk = which == 0 ? (H + kBlockCols - 1) / kBlockCols : (I + kBlockCols - 1) / kBlockCols;
    return nb * nk * kBlockRows * kBlockCols * 2;
}
hipError_t launch_pack_tile_blocks(int which, const void *w, int64_t E, int64_t I, int64_t H, void *out,
                                   hipStream_t st);

// Largest T*k for which the weight-streaming kernels route directly from the ids.
constexpr int kSkinnyDirectMax = 1024;
// Rows of one expert the weight-streaming kernels serve with its weights
// streamed once (two groups of 16 tokens per pass); in the mixed schedule,
// experts with more rows run on the tiled kernel.
constexpr int kSkinnyMaxRows = 32;

hipError_t launch_gate_up_tiled(const GemmProblem &p, hipStream_t st);
hipError_t launch_down_tiled(const GemmProblem &p, hipStream_t st);
hipError_t launch_gate_up_skinny(const GemmProblem &p, hipStream_t st);
hipError_t launch_down_skinny(const GemmProblem &p, hipStream_t st);
hipError_t launch_gate_up_f32(const GemmProblem &p, hipStream_t st);
hipError_t launch_down_f32(const GemmProblem &p, hipStream_t st);

int tiled_block_m();
int64_t tiled_split_bytes();  // partial-sum buffer of the large-M schedule
int tiled_tail_m();  // rows an expert's last M-tile may carry past tiled_block_m()

hipError_t launch_quantize_fp8_rows(const void *w, int64_t rows, int64_t cols, void *q, float *scale,
                                    hipStream_t st);
hipError_t launch_quantize_mxfp4_rows(const void *w, int64_t rows, int64_t cols, void *q, void *scale, hipStream_t st);

hipError_t launch_combine(const Shape &s, const float *slot, const float *sh_y, void *out,
                          hipStream_t st);

}  // namespace moe
