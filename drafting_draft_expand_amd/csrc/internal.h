// Host-side launch interfaces between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pe {

enum class DType { F32 = 0, BF16 = 1 };

// Best and runner-up logit over a set of vocabulary rows (ties -> lowest id).
struct Top2 {
  float v1;
  int i1;
  float v2;
  int pad;
};

inline int elem_bytes(DType t) { return t == DType::F32 ? 4 : 2; }

// Rotary inverse frequencies theta^(-2j/d), j < d/2 <= 64, formed on the host in
// double precision and passed by value in the kernel arguments.
struct RopeFreq {
  double inv[64];
};

// ---------------------------------------------------------------- expansion
struct PrepareArgs {
  int c, K, T, N, H, block_size, max_blocks, mask_id;
  int compact;                  // drop rejected rows (padding after the live rows)
  DType dtype;
  const int32_t *query_lens, *target_ids, *target_pos, *num_accepted, *bonus_ids, *block_table;
  const void *target_hidden, *h_shared;
  int32_t *draft_ids, *draft_pos;
  int64_t *slot_mapping;
  uint8_t *is_rejected, *is_masked;
  int32_t *hidden_map, *cu_draft, *kv_lens, *sample_idx;
  void *draft_hidden;
};
hipError_t launch_prepare(const PrepareArgs& a, hipStream_t s);

// Device-side check of the expansion's preconditions (bits as in peagle.h).
constexpr int kCheckQueryLen = 1, kCheckAccepted = 2, kCheckTokenId = 4, kCheckPosition = 8,
              kCheckBlockTable = 16;
struct CheckArgs {
  int c, K, T, V, max_blocks;
  const int32_t *query_lens, *target_ids, *target_pos, *num_accepted, *bonus_ids, *block_table;
  int32_t* error_bits;
};
hipError_t launch_check_batch(const CheckArgs& a, hipStream_t s);

// ---------------------------------------------------------------- projections
enum class Epi { Store = 0, AddTo = 1, SiluMul = 2, Argmax = 3, QkvRope = 4 };

// How the activation operand X[m, :] is formed.
enum class AMode {
  Plain = 0,   // X = x[m], model dtype, row stride K
  Gather = 1,  // X = [embed[ids[m]] ; x2[m]], each half K/2 elements (fc input)
  Norm = 2     // X = round(xf[r] / sqrt(mean(xf[r]^2) + eps) * gain), r = rows ? rows[m] : m;
               //     sum of xf[r]^2 = sum over t < ss_tiles of ss[t * ss_ld + r]
};

// Outputs of the fused q/k/v projection: rotate-half RoPE of q and k at the
// row's position, q stored as the attention operand, k/v written to the paged
// cache at the row's slot (nothing for slot -1).
struct RopeOut {
  int n_q, n_kv, d, block_size;
  const int64_t* slot;
  const uint8_t* rejected;
  void* q_out;                 // [M, n_q * d] model dtype
  void *k_cache, *v_cache;     // [blocks, n_kv, block_size, d]
  // [M][d / 2] (cos, sin) of row m's rotary angle j (its position times the
  // j-th inverse frequency, as rope_cos_sin evaluates them), written by the
  // RMSNorm before the projection; required
  const float2* table;
};

// Rotary table written by launch_rmsnorm: out[i][j] = (cos, sin) of
// pos[i] * freq.inv[j], j < half, for every row i (padding rows included).
struct RopeTable {
  const int32_t* pos;
  float2* out;
  int half;
  RopeFreq freq;
};

struct GemvArgs {
  // Y[m, n] = sum_k X[m, k] * W[n, k] for m < M, n < Nout.
  int M, Nout, K;
  // optional device count of live rows (rows at and past it are padding:
  // tiles that hold only padding rows are skipped); null: all M rows live
  const int32_t* m_live;
  AMode amode;
  const void* x;               // Plain
  const int32_t* ids;          // Gather
  const void *embed, *x2;      // Gather
  const float* xf;             // Norm
  const int32_t* rows;         // Norm (optional row gather)
  const void* gain;            // Norm
  const float* ss;             // Norm
  int ss_tiles, ss_ld;         // Norm
  float eps;                   // Norm
  // W rows: [0, n_a) from w_a, [n_a, n_a + n_b) from w_b, the rest from w_c;
  // every W row has K elements.  For Epi::SiluMul, w_a is the gate and w_b the
  // up projection (both Nout rows).
  const void *w_a, *w_b, *w_c;
  int n_a, n_b;
  // packed copies of the same rows in MFMA fragment order (PackArgs), used by
  // the weight-streaming MFMA kernel when set: pk_a for all Nout rows (the gate
  // for SiluMul), pk_b the up projection
  const void *pk_a, *pk_b;
  // tile-major copy of W for the ring GEMM: the LM head's rows in order
  // (launch_pack_tiles), or a layer projection's rows in the order its ring
  // tiles load them (launch_pack_proj_tiles); [rows / 256][K / 32][256][32]
  const void* pk_tiles;
  // x tile-major in groups of x_group rows ([M / G][K / 32][G][32], rows past M
  // present), 0: row-major; only with pk_tiles, and only G = 128
  int x_group;
  // outputs
  float* y;                    // Store / AddTo: fp32 [M, ldy]
  void* y_op;                  // SiluMul: model dtype [M, ldy]
  int ldy;
  // SiluMul: y_op tile-major in groups of y_group rows ([M / G][Nout / 32][G][32],
  // Nout % 32 == 0), 0: row-major; only G = 128
  int y_group;
  float* ss_out;               // Store / AddTo (MFMA kernel): [Nout / 16, M] row sums of y^2 per 16-column tile
  // Store / AddTo on packed weights without ss_out: when set, the kernel may
  // split K over `splits` workgroups and leave part[z][m][n] (stride ldy)
  // instead of writing y; the caller then forms y = (AddTo ? y : 0) + sum_z part[z]
  float* part;
  float* logits;               // Argmax: optional fp32 [M, Nout]
  Top2* partials;              // Argmax: [M, grid_x]
  RopeOut rope;                // QkvRope
  int grid_x;                  // filled by the launcher
  int splits;                  // filled by the launcher: K splits left in part (1: y written)
};
constexpr int kMaxSplits = 8;
// Kernel families: LDS-staged dot2 GEMV (fp32, and the bf16 LM head over at most
// 8 rows), weight-streaming MFMA (bf16, M <= 16), tiled MFMA GEMM (bf16, M > 16,
// K % 64 == 0).  The epilogue is that of the projection (argmax: the LM head).
enum class ProjKernel { Lds = 0, Skinny = 1, Tiled = 2 };
ProjKernel proj_kernel(int M, int K, DType dt, Epi epi = Epi::Store);
hipError_t launch_gemm(GemvArgs& a, Epi epi, int num_cus, hipStream_t s);
int gemm_parts(int M, int Nout, int num_cus);  // argmax candidates per row of the tiled kernel
hipError_t launch_gemv(GemvArgs& a, Epi epi, DType dt, int num_cus, hipStream_t s);
int gemv_grid_x(int M, int Nout, Epi epi, DType dt, int num_cus, int K);
size_t gemv_lds_bytes(int M, int K, DType dt, Epi epi = Epi::Store);  // dynamic LDS of the chosen kernel
bool gemv_uses_mfma(int M, int K, DType dt);

// Packed copy of W for the weight-streaming MFMA kernel: ceil(Nout / 16) tiles
// of K / 32 fragments; fragment (t, s) is 1 KiB at byte (t * K/32 + s) * 1024,
// its 16-byte piece l holding W[row(t, l % 16)][32 s + 8 (l / 16) .. + 8], row
// t*16 + c, or for rope_d > 0 the q/k/v order that puts rotary pairs (j, j+d/2)
// of one head in columns c and c + 8 of a tile.  Rows past Nout are zero.
struct PackArgs {
  void* dst;
  const void *w_a, *w_b, *w_c;  // rows [0, n_a), [n_a, n_a + n_b), the rest
  int n_a, n_b, Nout, K, rope_d;
};
size_t packed_bytes(int Nout, int K);
hipError_t launch_pack(const PackArgs& p, hipStream_t s);
// Tile-major copy of a row-major bf16 [Nout, K] matrix (K % 32 == 0) in
// 256-row groups, each 32-deep K step of a group one contiguous 16 KiB block.
size_t packed_tile_bytes(int Nout, int K);
hipError_t launch_pack_tiles(const void* w, int Nout, int K, void* dst, hipStream_t s);
// Tile-major copy of a layer projection for the ring GEMM over more than 256
// rows (Store / AddTo / SiluMul / QkvRope): packed row R holds the W row that
// row R % BN of the ring's N tile R / BN loads (q/k/v in rotary-pair order,
// gate and up rows interleaved as the SiluMul tile pairs them), in the layout
// of launch_pack_tiles.  `a` carries the W pointers and shape (w_a/w_b/w_c,
// n_a, n_b, Nout, K, rope.d).  The copy fits only the tile width the launcher
// uses for that epilogue over > 256 rows.
size_t proj_tile_bytes(Epi epi, int Nout, int K);
hipError_t launch_pack_proj_tiles(Epi epi, const GemvArgs& a, void* dst, hipStream_t s);

// ---------------------------------------------------------------- small kernels
hipError_t launch_build_fc_input(DType dt, int N, int H, const int32_t* ids, const void* embed,
                                 const void* draft_hidden, void* out, hipStream_t s);
// out[i] = RMSNorm(x[r]) * gain, r = row_idx ? row_idx[i] : i; H <= kMaxHidden.
// With nsplit > 0 the row is first completed from split partials and written
// back: x[r] = (accumulate ? x[r] : 0) + sum_z part[z][r] (z in order; split z
// starts at part + z * part_rows * H).  out_group > 0 (H % 32 == 0) writes out
// tile-major in groups of out_group rows: [rows / G][H / 32][G][32].
constexpr int kMaxHidden = 8192;
hipError_t launch_rmsnorm(DType dt, int rows, int H, const int32_t* row_idx, float* x, const void* gain,
                          float eps, void* out, hipStream_t s, const int32_t* live = nullptr,
                          const float* part = nullptr, int nsplit = 0, int part_rows = 0,
                          bool accumulate = false, int out_group = 0, const RopeTable* rope = nullptr);

struct RopeArgs {
  int N, n_q, n_kv, d, block_size;
  RopeFreq freq;
  DType dtype;
  const float* qkv;             // [N, (n_q + 2 n_kv) d]
  const int32_t* pos;
  const int64_t* slot;
  const uint8_t* rejected;
  void* q_out;                  // [N, n_q d] model dtype
  void *k_cache, *v_cache;      // [blocks, n_kv, block_size, d]
};
hipError_t launch_rope_kvwrite(const RopeArgs& a, hipStream_t s);

// Pages of one KV split that the bf16 MFMA attention keeps in LDS; with more
// (max_blocks > (kAttnMaxPages - 8) * splits) it reads the block table instead.
constexpr int kAttnMaxPages = 1088;
// KV-range splits per (sequence, kv head): at most this many
constexpr int kAttnMaxSplits = 16;

struct AttnArgs {
  int c, N, n_q, n_kv, d, block_size, max_blocks, splits;
  DType dtype;
  const void* q;                // [N, n_q d] model dtype (rotated)
  const int32_t* pos;
  const uint8_t* rejected;
  const int32_t *cu_draft, *kv_lens, *block_table;
  const void *k_cache, *v_cache;
  float* partial;               // [N, n_q, splits, d + 2]
  void* out;                    // [N, n_q d] model dtype
  // out tile-major in groups of out_group rows ([N / G][n_q d / 32][G][32],
  // n_q d % 32 == 0), 0: row-major
  int out_group;
  // every workgroup resident at once (the caller's estimate): launch slots
  // past the middle take the remaining sequences shortest first, so that the
  // two halves of the grid pair long with short
  int fold;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// Autoregressive baseline: store token k-1 and build the single row of pass k.
struct ArStepArgs {
  int c, K, k, H, max_blocks;
  bool last;                    // only store the final token
  DType dtype;
  const int32_t* prev_tokens;   // [c] tokens of pass k-1
  const float* x;               // residual rows of pass k-1 [rows, H]
  const int32_t* prev_sample_idx;  // rows of x that produced the tokens (null: row i)
  const int32_t* base_kv_lens;  // [c] kv lengths of the one-token first pass (= bonus position + 1)
  const int32_t* block_table;
  int32_t* draft_tokens;        // [c, K]
  int32_t *ids, *pos;
  int64_t* slot;
  uint8_t* rejected;
  int32_t *cu_draft, *kv_lens, *sample_idx;
  void* hidden;                 // [c, H] model dtype
};
hipError_t launch_ar_step(const ArStepArgs& a, hipStream_t s);
hipError_t launch_next_batch(int c, int K, const int32_t* kv_lens, const int32_t* bonus, const int32_t* drafts,
                             const int32_t* acc_next, const int32_t* bonus_next, int32_t* query_lens,
                             int32_t* target_ids, int32_t* target_pos, int32_t* num_accepted, int32_t* bonus_ids,
                             hipStream_t s);

hipError_t launch_argmax_finalize(int S, int parts, const Top2* partials, int32_t* tokens,
                                  float* gap, hipStream_t s);
hipError_t launch_accept(int c, int K, const int32_t* draft, const int32_t* target,
                         int32_t* acc, int32_t* bonus, hipStream_t s);

}  // namespace pe
