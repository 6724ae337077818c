// Tiled bf16 MFMA GEMM for many activation rows (M > 16): the drafter's
// projections at high concurrency and the LM head over c*K sampled rows.
//
// C[m, n] = sum_k A[m, k] * W[n, k], A and W both row-major with K contiguous.
// Four waves in a 2 x 2 grid per workgroup; each wave owns a WM x WN block of
// v_mfma_f32_16x16x32_bf16 tiles.  Per K step the next A/W tiles are fetched
// into registers while the current ones are read from LDS (16-byte chunks
// XOR-swizzled within each row, so fragment reads and staging writes are free
// of bank conflicts), then written to the other LDS buffer: one barrier per K
// step.  LDS traffic per MFMA falls as the wave block grows, so the largest
// tile that still gives every CU work is chosen: 128 x 256 (64 x 128 per
// wave) for the LM head and wide projections, smaller ones otherwise.
//
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so
// the logical tile index is taken from (blockIdx % 8, blockIdx / 8) such that
// the M tiles sharing one W tile run on the same XCD and reuse it from that
// XCD's L2 instead of fetching it from HBM once per M tile.
//
// Epilogues (same contracts as the weight-streaming kernels): store, residual
// add, SiLU(gate)*up (each wave's 8 N tiles are 4 gate + 4 matching up tiles),
// q/k/v with RoPE and the paged KV write (each 16-column MFMA tile holds 8
// rotary pairs, columns c and c^8), and LM-head argmax candidates per
// (row, 256-column tile).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace pe {
namespace {

// W row (global) loaded into B-tile row r of N tile nt.
template <Epi EPI, int BN, int WN>
__device__ __forceinline__ int b_row(const GemvArgs& a, int nt, int r) {
  if constexpr (EPI == Epi::SiluMul) {
    // BN/2 output columns per tile: wave column wn holds WN/2 gate rows then
    // the WN/2 matching up rows
    const int wn = r / WN, rr = r % WN;
    return nt * (BN / 2) + wn * (WN / 2) + (rr % (WN / 2));
  } else if constexpr (EPI == Epi::QkvRope) {
    const int col = nt * BN + r;
    const int per_head = a.rope.d / 16;
    const int t = col / 16, c = col % 16;
    const int head = t / per_head, p = t - head * per_head;
    return head * a.rope.d + 8 * p + (c & 7) + (c >= 8 ? a.rope.d / 2 : 0);
  } else {
    return nt * BN + r;
  }
}

template <Epi EPI, int BN, int WN>
__device__ __forceinline__ const bf16_t* b_ptr(const GemvArgs& a, int nt, int r) {
  const int K = a.K;
  const int n = min(b_row<EPI, BN, WN>(a, nt, r), a.Nout - 1);
  if constexpr (EPI == Epi::SiluMul) {
    return static_cast<const bf16_t*>((r % WN) < WN / 2 ? a.w_a : a.w_b) + static_cast<int64_t>(n) * K;
  } else {
    if (n < a.n_a) return static_cast<const bf16_t*>(a.w_a) + static_cast<int64_t>(n) * K;
    if (n < a.n_a + a.n_b) return static_cast<const bf16_t*>(a.w_b) + static_cast<int64_t>(n - a.n_a) * K;
    return static_cast<const bf16_t*>(a.w_c) + static_cast<int64_t>(n - a.n_a - a.n_b) * K;
  }
}

// Element offset of 16-byte chunk c of LDS tile row r (rows of CPR chunks,
// unpadded).  Chunks are XOR-swizzled within the row -- c ^ (r & 7) for
// 128-byte rows, c ^ ((r >> 1) & 3) for 64-byte rows -- so that both the
// staging writes (consecutive lanes along a row) and the MFMA fragment reads
// (16 rows, 4 chunks) of ds_read_b128 / ds_write_b128 hit distinct banks.
template <int CPR>
__device__ __forceinline__ int lds_off(int r, int c) {
  const int sw = CPR == 8 ? (c ^ (r & 7)) : (c ^ ((r >> 1) & 3));
  return r * (CPR * 8) + sw * 8;
}

// Epilogue of one output tile held in MFMA accumulators: wave (wm, wn) of a
// WGM x WGN wave grid owns rows m0 + wm * 16 TM .. and tile columns
// wn * 16 TN ..; lane l holds rows 4 (l / 16) + q, column l % 16 of each
// 16 x 16 block.  red is LDS scratch for WGN * BM candidates (argmax only).
template <int BM, int BN, int WGM, int WGN, int TM, int TN, Epi EPI>
__device__ __forceinline__ void tile_epilogue(const GemvArgs& a, f32x4 (&acc)[TM][TN], int m0, int nt, int num_n,
                                              int wm, int wn, Top2* red, int z, int splits) {
  constexpr int WM = TM * 16, WN = TN * 16, NT = WGM * WGN * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  if constexpr (EPI == Epi::Store || EPI == Epi::AddTo) {
    // K split over workgroups: the sum of this split goes to part[z]
    float* out = splits > 1 ? a.part + static_cast<int64_t>(z) * a.M * a.ldy : a.y;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) {
        const int n = nt * BN + wn * WN + jn * 16 + l16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + wm * WM + i * 16 + lq * 4 + q;
          if (m >= a.M || n >= a.Nout) continue;
          float* y = out + static_cast<int64_t>(m) * a.ldy + n;
          if (EPI == Epi::AddTo && splits == 1) *y += acc[i][jn][q];
          else *y = acc[i][jn][q];
        }
      }
  } else if constexpr (EPI == Epi::SiluMul) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < TN / 2; ++jn) {
        const int n = nt * (BN / 2) + wn * (WN / 2) + jn * 16 + l16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + wm * WM + i * 16 + lq * 4 + q;
          if (m >= a.M || n >= a.Nout) continue;
          const float gt = acc[i][jn][q];
          const float sg = gt / (1.f + expf(-gt));
          // row-major, or tile-major in 128-row groups for a consumer that
          // reads its A operand that way
          const int64_t at = a.y_group ? (static_cast<int64_t>(m >> 7) * a.Nout + (n & ~31)) * 128 + (m & 127) * 32 +
                                             (n & 31)
                                       : static_cast<int64_t>(m) * a.ldy + n;
          static_cast<bf16_t*>(a.y_op)[at] = f32_to_bf16(sg * acc[i][jn + TN / 2][q]);
        }
      }
  } else if constexpr (EPI == Epi::QkvRope) {
    const RopeOut& ro = a.rope;
    const int d = ro.d;  // 16, 32, 64 or 128
    const int ld = 31 - __builtin_clz(d);
    const int half = d >> 1;
    // column facts once (they do not depend on the row): output head and
    // element of each of this lane's columns
    int c_head[TN], c_e[TN];
    bool c_ok[TN];
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) {
      const int n = b_row<EPI, BN, WN>(a, nt, wn * WN + jn * 16 + l16);
      c_head[jn] = n >> ld;
      c_e[jn] = n & (d - 1);
      c_ok[jn] = nt * BN + wn * WN + jn * 16 + l16 < a.Nout;
    }
    // Phase 1: rotate the accumulators in place, 16 rows at a time: with no
    // store in between, each group's table entries are waited for once
    // (stores count in the same in-order counter as loads, so a table read
    // issued after a store would have to wait for that store too).
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float2 tv[4][TN];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mc = min(m0 + wm * WM + i * 16 + lq * 4 + q, a.M - 1);
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
          tv[q][jn] = ro.table[static_cast<int64_t>(mc) * half + (c_e[jn] & (half - 1))];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
          const float v = acc[i][jn][q];
          const float partner = __shfl_xor(v, 8, 64);
          if (c_head[jn] < ro.n_q + ro.n_kv)
            acc[i][jn][q] = (l16 & 8) == 0 ? v * tv[q][jn].x - partner * tv[q][jn].y
                                            : v * tv[q][jn].x + partner * tv[q][jn].y;
        }
    }
    // Phase 2: stores.  Row facts (rejected flag, cache slot) requested in one
    // batch at clamped rows.
    uint8_t r_rej[TM * 4];
    int64_t r_slot[TM * 4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mc = min(m0 + wm * WM + i * 16 + lq * 4 + q, a.M - 1);
        r_rej[i * 4 + q] = ro.rejected[mc];
        r_slot[i * 4 + q] = ro.slot[mc];
      }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * WM + i * 16 + lq * 4 + q;
        if (m >= a.M || r_rej[i * 4 + q]) continue;
        const int64_t slot = r_slot[i * 4 + q];
        // 16-token pages (the only page size the library accepts)
        const int64_t page_row = slot < 0 ? 0 : ((slot >> 4) * ro.n_kv * 16 + (slot & 15)) << ld;
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
          if (!c_ok[jn]) continue;
          const int head = c_head[jn], e = c_e[jn];
          const bf16_t out = f32_to_bf16(acc[i][jn][q]);
          if (head < ro.n_q) {
            static_cast<bf16_t*>(ro.q_out)[((static_cast<int64_t>(m) * ro.n_q + head) << ld) + e] = out;
          } else if (slot >= 0) {
            const bool is_k = head < ro.n_q + ro.n_kv;
            const int g = is_k ? head - ro.n_q : head - ro.n_q - ro.n_kv;
            static_cast<bf16_t*>(is_k ? ro.k_cache : ro.v_cache)[page_row + (static_cast<int64_t>(g) << (4 + ld)) + e] =
                out;
          }
        }
      }
  } else {  // Argmax over this tile's BN columns, per row
    if (a.logits) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
          const int n = nt * BN + wn * WN + jn * 16 + l16;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = m0 + wm * WM + i * 16 + lq * 4 + q;
            if (m < a.M && n < a.Nout) a.logits[static_cast<int64_t>(m) * a.Nout + n] = acc[i][jn][q];
          }
        }
    }
    // Each lane's TM * 4 rows: the candidates of its TN columns merged
    // pairwise (a column past Nout adds nothing) ...
    static_assert(TM == 4 && (TN & (TN - 1)) == 0, "16 rows per lane, a power-of-two column count");
    Top2 t[16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Top2 c[TN];
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
          const int n = nt * BN + wn * WN + jn * 16 + l16;
          // one column as a candidate set: itself, or nothing if it lies
          // past Nout or is NaN (what pushing it into an empty set gives)
          const float v = acc[i][jn][q];
          const bool ok = n < a.Nout && v == v;
          c[jn] = top2_empty();
          c[jn].v1 = ok ? v : c[jn].v1;
          c[jn].i1 = ok ? n : c[jn].i1;
        }
#pragma unroll
        for (int w = 1; w < TN; w *= 2)
#pragma unroll
          for (int jn = 0; jn < TN; jn += 2 * w) c[jn] = top2_merge(c[jn], c[jn + w]);
        t[i * 4 + q] = c[0];
      }
    // ... then exchanged over the 16 lanes that hold the same rows: at
    // distance o a lane keeps the half of its o * 2 rows that bit o of its
    // lane index selects and merges in its partner's candidates for that
    // half, so after four steps lane l16 holds row l16 (i = l16 / 4,
    // q = l16 % 4) merged over all 16 lanes.  The merge result does not
    // depend on the order (best value, lowest id on ties; runner-up = largest
    // of the rest), so this equals the row-by-row reduction.
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const bool up = (l16 & o) != 0;
#pragma unroll
      for (int r = 0; r < o; ++r) {
        const Top2 keep = up ? t[r + o] : t[r];
        const Top2 give = up ? t[r] : t[r + o];
        Top2 got;
        got.v1 = __shfl_xor(give.v1, o, 64);
        got.i1 = __shfl_xor(give.i1, o, 64);
        got.v2 = __shfl_xor(give.v2, o, 64);
        got.pad = 0;
        t[r] = top2_merge(keep, got);
      }
    }
    red[wn * BM + wm * WM + (l16 >> 2) * 16 + lq * 4 + (l16 & 3)] = t[0];
    __syncthreads();
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      Top2 t = red[r];
#pragma unroll
      for (int w = 1; w < WGN; ++w) t = top2_merge(t, red[w * BM + r]);
      if (m < a.M) a.partials[static_cast<int64_t>(m) * num_n + nt] = t;
    }
  }
}

template <int BM, int BN, int BK, int PD, int WGM, Epi EPI, AMode MODE>
__global__ __launch_bounds__(256, BM * BN >= 256 * 256 ? 1 : 2) void gemm_kernel(GemvArgs a, int num_m, int num_n,
                                                                                  int splits) {
  constexpr int WGN = 4 / WGM;                // wave grid WGM x WGN
  constexpr int WM = BM / WGM, WN = BN / WGN; // wave block
  constexpr int TM = WM / 16, TN = WN / 16;   // MFMA tiles per wave
  constexpr int LDT = BK;                     // LDS row, elements (no padding: chunks are swizzled)
  constexpr int CPR = BK / 8;                 // 16-byte chunks per tile row
  static_assert(CPR == 4 || CPR == 8, "K step 32 or 64");
  constexpr int NA = (BM * CPR + 255) / 256, NB = (BN * CPR + 255) / 256;  // chunks per thread
  static_assert(NA >= 1 && NB >= 1, "tile too small");
  static_assert(PD == 1 || PD == 2 || PD == 4, "prefetch distance 1, 2 or 4");
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDT];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  // XCD-aware tile order: the M tiles of one (W tile, K split) land on one XCD
  const int total = num_m * num_n * splits;
  const int per_xcd = (total + 7) / 8;
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L >= total) return;
  const int mt = L % num_m, rest = L / num_m;
  const int z = rest % splits, nt = rest / splits;
  const int m0 = mt * BM;
  if (a.m_live && m0 >= *a.m_live) return;  // only padding rows in this tile
  // this workgroup's K steps: [kbase, kbase + nk) of the K / BK steps
  const int nk_all = a.K / BK;
  const int per_split = (nk_all + splits - 1) / splits;
  const int kbase = min(nk_all, z * per_split);
  const int nk = min(nk_all, kbase + per_split) - kbase;

  // thread -> 16-byte chunk mapping of the A and W tiles (rows of CPR chunks);
  // recomputed where used rather than held in registers
  const int c_row = tid / CPR, c_col = (tid % CPR) * 8;
  constexpr int ROWS_PER_PASS = 256 / CPR;
  const bf16_t* bp0 = b_ptr<EPI, BN, WN>(a, nt, c_row) + c_col;
  // W rows of one pass are consecutive except where a segment or the gate/up
  // pairing switches; those cases take the general pointer per chunk.
  constexpr bool W_CONTIG = EPI == Epi::Store || EPI == Epi::AddTo || EPI == Epi::Argmax;
  // Global loads run PD K steps ahead of the MFMAs: tile t waits in register
  // set t % PD and is consumed from LDS buffer t & 1; the K loop is unrolled by
  // max(PD, 2) so every set and buffer index is a compile-time constant (no
  // indexed register access).
  u32x4 ra[PD][NA], rb[PD][NB];
  // A source rows, resolved once (for the gathered operand: the token's
  // embedding row and the row's draft hidden state, each K/2 wide)
  const bf16_t* ap0[NA];
  const bf16_t* ap1[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int m = min(m0 + c_row + i * ROWS_PER_PASS, a.M - 1);
    if constexpr (MODE == AMode::Gather) {
      const int half = a.K / 2;
      ap0[i] = static_cast<const bf16_t*>(a.embed) + static_cast<int64_t>(a.ids[m]) * half + c_col;
      ap1[i] = static_cast<const bf16_t*>(a.x2) + static_cast<int64_t>(m) * half + c_col - half;
    } else {
      ap0[i] = static_cast<const bf16_t*>(a.x) + static_cast<int64_t>(m) * a.K + c_col;
      ap1[i] = ap0[i];
    }
  }
  auto fetch = [&](int kt, auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    const int k0 = (kbase + kt) * BK;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if ((BM * CPR) % 256 == 0 || c_row + i * ROWS_PER_PASS < BM) {
        const bool lo = MODE != AMode::Gather || k0 + c_col < a.K / 2;
        ra[set][i] = load16((lo ? ap0[i] : ap1[i]) + k0);
      }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = c_row + i * ROWS_PER_PASS;
      if ((BN * CPR) % 256 != 0 && r >= BN) continue;
      const bf16_t* p = W_CONTIG && b_row<EPI, BN, WN>(a, nt, r) < a.n_a
                            ? bp0 + static_cast<int64_t>(i * ROWS_PER_PASS) * a.K
                            : b_ptr<EPI, BN, WN>(a, nt, r) + c_col;
      rb[set][i] = load16(p + k0);
    }
  };
  auto stash = [&](auto buf_c, auto set_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value, set = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r = c_row + i * ROWS_PER_PASS;
      if ((BM * CPR) % 256 == 0 || r < BM) store16(&As[buf][lds_off<CPR>(r, c_col / 8)], ra[set][i]);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = c_row + i * ROWS_PER_PASS;
      if ((BN * CPR) % 256 == 0 || r < BN) store16(&Bs[buf][lds_off<CPR>(r, c_col / 8)], rb[set][i]);
    }
  };
  using C0 = std::integral_constant<int, 0>;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15, lq = lane >> 4;
  auto compute = [&](auto buf_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(buf_c)::value;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      // all W fragments of the K slice stay in registers; A fragments are
      // read one at a time so the live set stays small
      u32x4 bf[TN];
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
        bf[jn] = *reinterpret_cast<const u32x4*>(&Bs[cur][lds_off<CPR>(wn * WN + jn * 16 + l16, ks * 4 + lq)]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(&As[cur][lds_off<CPR>(wm * WM + i * 16 + l16, ks * 4 + lq)]);
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                               __builtin_bit_cast(bf16x8, bf[jn]), acc[i][jn], 0, 0,
                                                               0);
      }
    }
  };
  // One K step: compute from LDS buffer kt & 1, publish tile kt+1 (register
  // set (kt+1) % PD) in the other buffer, request tile kt+1+PD into that set.
  // Publishing and requesting are unconditional -- past the last tile they
  // re-request the last tile (cache hits) and publish into a buffer nobody
  // reads -- so the steady state has no branches and the compiler's counters
  // of outstanding loads stay exact: publishing tile kt+1 waits only for its
  // own loads, with the PD-1 younger tiles still in flight.
  auto step = [&](int kt, auto buf_c, auto setn_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(buf_c)::value;
    using Nxt = std::integral_constant<int, cur ^ 1>;
    compute(buf_c);
    stash(Nxt{}, setn_c);
    fetch(min(kt + 1 + PD, nk - 1), setn_c);
    __syncthreads();
  };

  // prologue: tiles 0 .. PD-1 requested into sets 0 .. PD-1 (clamped to the
  // split's last tile; every split has at least one: splits <= K / BK), tile 0
  // published, tile PD requested into the set tile 0 freed
  static_for<PD>([&](auto j_c) { fetch(min(static_cast<int>(decltype(j_c)::value), nk - 1), j_c); });
  stash(C0{}, C0{});
  fetch(min(PD, nk - 1), C0{});
  __syncthreads();
  // whole unrolled blocks without branches, then the remaining steps
  constexpr int UN = PD == 1 ? 2 : PD;
  const int nk_main = nk - nk % UN;
  for (int kt = 0; kt < nk_main; kt += UN) {
    static_for<UN>([&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      step(kt + j, std::integral_constant<int, j & 1>{}, std::integral_constant<int, (j + 1) % PD>{});
    });
  }
  static_for<UN - 1>([&](auto j_c) {
    constexpr int j = decltype(j_c)::value;
    if (nk_main + j < nk)
      step(nk_main + j, std::integral_constant<int, j & 1>{}, std::integral_constant<int, (j + 1) % PD>{});
  });

  // ---------------------------------------------------------------- epilogue
  static_assert(WGN * BM * sizeof(Top2) <= sizeof(Bs) / 2, "argmax scratch must fit one LDS buffer");
  tile_epilogue<BM, BN, WGM, WGN, TM, TN, EPI>(a, acc, m0, nt, num_n, wm, wn, reinterpret_cast<Top2*>(&Bs[0][0]), z,
                                               splits);
}

// ------------------------------------------------------------- LDS-DMA ring
// The same tiles fed by direct global -> LDS copies (global_load_lds_dwordx4)
// into a ring of ST LDS stages, one 32-deep K step each (or two: 64-deep
// stages); no register staging.  A wave's copy instruction writes one
// contiguous KiB of LDS, 16 tile rows of 64 bytes, lane l landing in row
// l / 4, chunk l % 4 (64-deep: 8 rows of 128 bytes, row l / 8, chunk l % 8);
// the lane fetches the global chunk that the row's XOR swizzle places there,
// so the fragment reads are the register-staged kernel's.
//
// Operand layouts.  Row-major, a copy instruction gathers 16 rows x 64 bytes;
// tile-major ("packed": [rows / G][K / 32][G][32], G = 256 for W, BM for A,
// each K step of a row group one contiguous block) it reads one contiguous
// KiB.  On this GPU the contiguous form keeps the L2 -> LDS path about 10-20%
// busier for the LM head over 448 rows (measured 0.31-0.33 of bf16 peak
// row-major, 0.37-0.44 with both operands packed).
//
// Synchronisation is explicit (the compiler does not track these LDS
// writes).  Without fragment prefetch (PF false), step t waits until its own
// copies of stage t have landed and its LDS reads of step t-1 are done
// (s_waitcnt with ST-2 stages still in flight), one barrier makes that hold
// for the whole workgroup, then the wave requests step t+ST-1 into the slot
// step t-1 used and multiplies.  With PF, the fragments of step t+1 are read
// from LDS while step t's MFMAs run: at the end of step t the wave waits for
// stage t+2 and for its reads, and the barrier publishes stage t+2 and frees
// slot t+1's predecessor; step t then requests step t+ST into slot t, whose
// fragments are already in registers.  Requests past the split's last step
// re-read that step (cache hits) so the steady state has no branches.

// Row group of the tile-major W copy (packed_tile_bytes / launch_pack_tiles).
constexpr int kTileGroup = 256;

template <int BM, int BN, int ST, bool PF, bool PKA, bool PKW, Epi EPI, int BKS = 32, bool GA = false>
__global__ __launch_bounds__(256, ST * (BM + BN) * BKS * 2 > 80 * 1024 ? 1 : 2) void gemm_ring_kernel(GemvArgs a,
                                                                                                   int num_m, int num_n,
                                                                                                   int splits) {
  // BKS: K depth of one stage.  32: a copy instruction moves 16 tile rows of
  // 64 bytes; 64: 8 rows of 128 bytes (whole cache lines of row-major
  // operands, two MFMA K steps per stage; row-major operands, no prefetch).
  constexpr int BK = BKS, CPR = BK / 8, KK = BK / 32, RPC = 512 / BK, WGM = 2, WGN = 2;
  static_assert(BK == 32 || (BK == 64 && !PF && !PKA && !PKW), "64-deep stages: row-major operands, no prefetch");
  // GA: the A rows are gathered, [embed[ids[m]] ; x2[m]] (K / 2 elements
  // each, K / 2 a multiple of the stage depth), as the fc input
  static_assert(!GA || (!PKA && !PF), "gathered A rows are row-major");
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  // PKW: the tile-major copy holds W rows in the order the N tiles load them
  // (plain for the LM head, Store and AddTo; launch_pack_proj_tiles for all)
  static_assert(BM % (4 * RPC) == 0 && BN % (4 * RPC) == 0, "whole copy blocks for every wave");
  static_assert(!PKW || kTileGroup % BN == 0, "a W tile lies inside one packed row group");
  constexpr int IA = BM / (4 * RPC), IB = BN / (4 * RPC);  // copy instructions per wave and stage
  constexpr int NI = IA + IB;
  static_assert(ST >= 3 && (ST - 2) * NI <= 63, "outstanding copy count must fit the counter");
  static_assert(WGN * BM * sizeof(Top2) <= sizeof(bf16_t) * (BM + BN) * BK, "argmax scratch must fit one ring stage");
  // One LDS variable per ring stage (A rows then W rows) so every stage is
  // addressed by a compile-time constant.
  constexpr int SZ = (BM + BN) * BK;
  __shared__ __attribute__((aligned(16))) bf16_t R0[SZ];
  __shared__ __attribute__((aligned(16))) bf16_t R1[SZ];
  __shared__ __attribute__((aligned(16))) bf16_t R2[SZ];
  __shared__ __attribute__((aligned(16))) bf16_t R3[ST > 3 ? SZ : 8];
  __shared__ __attribute__((aligned(16))) bf16_t R4[ST > 4 ? SZ : 8];
  static_assert(ST <= 5, "at most five ring stages");
  auto ring = [&](auto s_c) __attribute__((always_inline)) -> bf16_t* {
    constexpr int S = decltype(s_c)::value % ST;
    if constexpr (S == 0) return R0;
    else if constexpr (S == 1) return R1;
    else if constexpr (S == 2) return R2;
    else if constexpr (S == 3) return R3;
    else return R4;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int total = num_m * num_n * splits;
  const int per_xcd = (total + 7) / 8;
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L >= total) return;
  const int mt = L % num_m, rest = L / num_m;
  const int z = rest % splits, nt = rest / splits;
  const int m0 = mt * BM;
  // A tile of padding rows only (compacted layout) stops once its first copies
  // have landed.  The live count is read (scalar load) just before the first
  // copies are requested and tested after them, so that live tiles do not
  // wait for it first; read after the copies (which clobber memory as far as
  // the compiler knows) it would become a vector load whose wait drains them.
  int live_rows = 0x7fffffff;
  auto read_live = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if (a.m_live) live_rows = *a.m_live;
  };
  auto padding_tile = [&]() __attribute__((always_inline)) { return m0 >= live_rows; };
  const int nk_all = a.K / BK;
  const int per_split = (nk_all + splits - 1) / splits;
  const int kbase = min(nk_all, z * per_split);
  const int nk = min(nk_all, kbase + per_split) - kbase;

  // this lane's source chunk in each of the wave's copy blocks, at K step 0,
  // and the element stride from one K step to the next
  const int lrow = lane / CPR;
  // global chunk that the row's swizzle (lds_off) places in this lane's slot
  auto chunk_of = [&](int r) { return CPR == 8 ? (lane & 7) ^ (r & 7) : (lane & 3) ^ ((r >> 1) & 3); };
  const bf16_t* ap[IA];
  const bf16_t* ap_hi[GA ? IA : 1];  // GA: the second half's rows, offset by -K / 2
#pragma unroll
  for (int q = 0; q < IA; ++q) {
    const int r = (q * 4 + wave) * RPC + lrow;
    const int gc = chunk_of(r);
    if constexpr (GA) {
      const int m = min(m0 + r, a.M - 1), half = a.K / 2;
      ap[q] = static_cast<const bf16_t*>(a.embed) + static_cast<int64_t>(a.ids[m]) * half + gc * 8;
      ap_hi[q] = static_cast<const bf16_t*>(a.x2) + static_cast<int64_t>(m) * half + gc * 8 - half;
    } else if constexpr (PKA)
      ap[q] = static_cast<const bf16_t*>(a.x) + (static_cast<int64_t>(mt) * nk_all * BM + r) * BK + gc * 8;
    else
      ap[q] = static_cast<const bf16_t*>(a.x) + static_cast<int64_t>(min(m0 + r, a.M - 1)) * a.K + gc * 8;
  }
  const bf16_t* bp[IB];
#pragma unroll
  for (int q = 0; q < IB; ++q) {
    const int r = (q * 4 + wave) * RPC + lrow;
    const int gc = chunk_of(r);
    if constexpr (PKW) {
      const int row = nt * BN + r;  // rows past Nout exist in the packed copy
      bp[q] = static_cast<const bf16_t*>(a.pk_tiles) +
              ((static_cast<int64_t>(row / kTileGroup) * nk_all) * kTileGroup + row % kTileGroup) * BK + gc * 8;
    } else {
      bp[q] = b_ptr<EPI, BN, WN>(a, nt, r) + gc * 8;
    }
  }
  constexpr int64_t A_STEP = PKA ? BM * BK : BK, B_STEP = PKW ? kTileGroup * BK : BK;
  // The LM head over at most 128 rows (the instance without fragment
  // prefetch) has one M tile, so each W tile is read exactly once: its copies
  // are non-temporal and leave the caches to the rows (Qwen-shaped head over
  // 112 rows: step 0.378-0.385 -> 0.351-0.357 ms).  With several M tiles (and
  // in the layer projections) the W tiles are shared through L2 and keep the
  // default policy.
  constexpr bool W_STREAM = PKW && !PF && EPI == Epi::Argmax;
  auto request = [&](int kt, auto s_c) __attribute__((always_inline)) {
    bf16_t* st = ring(s_c);
    const int64_t k = kbase + min(kt, nk - 1);
#pragma unroll
    for (int q = 0; q < IA; ++q) {
      const bf16_t* src = ap[q];
      if constexpr (GA) src = k * BK < a.K / 2 ? ap[q] : ap_hi[q];  // the same half for the whole stage
      dma16(src + k * A_STEP, st + (q * 4 + wave) * RPC * BK);
    }
#pragma unroll
    for (int q = 0; q < IB; ++q) dma16<W_STREAM>(bp[q] + k * B_STEP, st + BM * BK + (q * 4 + wave) * RPC * BK);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int l16 = lane & 15, lq = lane >> 4;
  constexpr int NF = PF ? 2 : 1;  // fragment sets
  u32x4 fa[NF][KK][TM], fb[NF][KK][TN];
  auto frags = [&](auto s_c, auto f_c) __attribute__((always_inline)) {
    constexpr int F = decltype(f_c)::value;
    const bf16_t* as = ring(s_c);
    const bf16_t* bs = as + BM * BK;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
        fb[F][kk][jn] = *reinterpret_cast<const u32x4*>(&bs[lds_off<CPR>(wn * WN + jn * 16 + l16, kk * 4 + lq)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[F][kk][i] = *reinterpret_cast<const u32x4*>(&as[lds_off<CPR>(wm * WM + i * 16 + l16, kk * 4 + lq)]);
    }
  };
  auto mma = [&](auto f_c) __attribute__((always_inline)) {
    constexpr int F = decltype(f_c)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[F][kk][i]),
                                                               __builtin_bit_cast(bf16x8, fb[F][kk][jn]), acc[i][jn], 0, 0,
                                                               0);
  };
  // wait until at most ST-2 stages of copies are in flight and no LDS read
  // is, then meet the other waves
  constexpr int kWait = waitcnt_vm_lgkm0((ST - 2) * NI);
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWait);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  using C0 = std::integral_constant<int, 0>;

  if constexpr (PF) {
    // A wave whose rows all lie past M (the last M tile of a row count that
    // is not a multiple of BM) still issues its share of the copies and meets
    // every barrier, but reads no fragments and runs no MFMAs: its SIMD goes
    // to the other workgroup on the CU.  Its accumulators stay zero, and the
    // epilogue writes no row past M.
    auto run = [&](auto live_c) __attribute__((always_inline)) -> bool {
      constexpr bool LIVE = decltype(live_c)::value;
      // prologue: steps 0 .. ST-1 requested, stages 0 and 1 landed
      // everywhere, step 0's fragments in registers and every wave done
      // reading slot 0
      read_live();
      static_for<ST>([&](auto s_c) { request(decltype(s_c)::value, s_c); });
      if (padding_tile()) {
        __builtin_amdgcn_s_waitcnt(0);
        return false;
      }
      sync();
      if constexpr (LIVE) frags(C0{}, C0{});
      sync();
      auto step = [&](int t, auto j_c) __attribute__((always_inline)) {
        constexpr int J = decltype(j_c)::value;
        request(t + ST, std::integral_constant<int, J % ST>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LIVE) {
          frags(std::integral_constant<int, (J + 1) % ST>{}, std::integral_constant<int, (J + 1) & 1>{});
          mma(std::integral_constant<int, J & 1>{});
          // one fragment read, then two MFMAs, ..., then the remaining MFMAs
          static_for<TM + TN>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          });
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - 2 * (TM + TN), 0);
        }
        sync();
      };
      constexpr int U = ST % 2 == 0 ? ST : 2 * ST;
      int t = 0;
      for (; t + U <= nk; t += U) static_for<U>([&](auto j_c) { step(t + decltype(j_c)::value, j_c); });
      static_for<U - 1>([&](auto j_c) {
        if (t + decltype(j_c)::value < nk) step(t + decltype(j_c)::value, j_c);
      });
      return true;
    };
    const bool go = m0 + wm * WM < a.M ? run(std::true_type{}) : run(std::false_type{});
    if (!go) return;
  } else {
    read_live();
    static_for<ST - 1>([&](auto s_c) { request(decltype(s_c)::value, s_c); });
    if (padding_tile()) {
      __builtin_amdgcn_s_waitcnt(0);
      return;
    }
    auto step = [&](int t, auto s_c) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value;
      sync();
      request(t + ST - 1, std::integral_constant<int, (S + ST - 1) % ST>{});
      frags(s_c, C0{});
      mma(C0{});
    };
    int t = 0;
    for (; t + ST <= nk; t += ST) static_for<ST>([&](auto s_c) { step(t + decltype(s_c)::value, s_c); });
    static_for<ST - 1>([&](auto s_c) {
      if (t + decltype(s_c)::value < nk) step(t + decltype(s_c)::value, s_c);
    });
  }
  // every copy (the clamped requests past the end included) has landed and
  // every LDS read is done before the epilogue reuses slot 0
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  tile_epilogue<BM, BN, WGM, WGN, TM, TN, EPI>(a, acc, m0, nt, num_n, wm, wn, reinterpret_cast<Top2*>(R0), z, splits);
}

int gemm_splits(const GemvArgs& a, Epi epi, int tiles, int nk_all, int num_cus);

template <int BM, int BN, int ST, bool PF, bool PKA, bool PKW, Epi EPI, int BKS = 32, bool GA = false>
hipError_t launch_ring(GemvArgs& a, int num_cus, hipStream_t s) {
  const int num_m = (a.M + BM - 1) / BM;
  const int cols = EPI == Epi::SiluMul ? BN / 2 : BN;  // gate + up rows per output column
  const int num_n = (a.Nout + cols - 1) / cols;
  if (a.K % BKS != 0 || (GA && (a.K / 2) % BKS != 0)) return hipErrorInvalidValue;
  const int splits = gemm_splits(a, EPI, num_m * num_n, a.K / BKS, num_cus);
  const int total = num_m * num_n * splits;
  const int grid = ((total + 7) / 8) * 8;
  a.grid_x = num_n;
  a.splits = splits;
  hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, ST, PF, PKA, PKW, EPI, BKS, GA>), dim3(grid), dim3(256), 0, s, a,
                     num_m, num_n, splits);
  return hipGetLastError();
}

// Tile shapes (K step 32 for the 256-column tile, 64 for the others; loads
// run two K steps ahead for all three).
struct TileCfg {
  int bm, bn;
};
constexpr TileCfg kLarge{128, 256}, kMedium{128, 128}, kSmall{128, 64};

int cols_per_tile(const TileCfg& t, Epi epi) { return epi == Epi::SiluMul ? t.bn / 2 : t.bn; }
int tiles_of(const TileCfg& t, int M, int Nout, Epi epi) {
  const int c = cols_per_tile(t, epi);
  return ((M + t.bm - 1) / t.bm) * ((Nout + c - 1) / c);
}

// Largest tile that still fills the chip: the 256-column tile when there are
// several M tiles to share each W tile in L2 and a workgroup per CU, the
// 128-column tile with two workgroups per CU, else the 64-column tile.
TileCfg pick_tile(int M, int Nout, Epi epi, int num_cus) {
  // (the q/k/v epilogue does not fit the 256-column tile's registers)
  if (M > 128 && epi != Epi::QkvRope && tiles_of(kLarge, M, Nout, epi) >= num_cus) return kLarge;
  if (tiles_of(kMedium, M, Nout, epi) >= 2 * num_cus) return kMedium;
  return kSmall;
}

// K splits for Store / AddTo when the tiles alone leave CUs idle and the
// caller takes partial sums.  One workgroup per CU when that still splits K at
// least twice, else as many as fit in one round of two per CU: what matters is
// the busiest CU's share, and a count just past a round boundary doubles it
// (552 units over 512 slots ran 10-15% slower than 414).  Fewer splits also
// leave fewer partial sums for the next RMSNorm to read (at 672 rows, 3
// splits instead of 7 for o / down: the same GEMM time, 2.4 us less per norm).
// At most kMaxSplits and at least 8 K steps per split.
int gemm_splits(const GemvArgs& a, Epi epi, int tiles, int nk_all, int num_cus) {
  if (!a.part || a.ss_out || (epi != Epi::Store && epi != Epi::AddTo)) return 1;
  int sp = num_cus / tiles >= 2 ? num_cus / tiles : 2 * num_cus / tiles;
  if (sp > kMaxSplits) sp = kMaxSplits;
  if (sp > nk_all / 8) sp = nk_all / 8;
  return sp < 2 ? 1 : sp;
}

template <int BM, int BN, int BK, int PD, int WGM, Epi EPI, AMode MODE>
hipError_t launch_t(GemvArgs& a, int num_cus, hipStream_t s) {
  const int num_m = (a.M + BM - 1) / BM;
  const int cols = EPI == Epi::SiluMul ? BN / 2 : BN;
  const int num_n = (a.Nout + cols - 1) / cols;
  const int splits = gemm_splits(a, EPI, num_m * num_n, a.K / BK, num_cus);
  const int total = num_m * num_n * splits;
  const int grid = ((total + 7) / 8) * 8;
  a.grid_x = num_n;
  a.splits = splits;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, PD, WGM, EPI, MODE>), dim3(grid), dim3(256), 0, s, a, num_m, num_n,
                     splits);
  return hipGetLastError();
}

// 17..256 rows: the LDS-DMA ring on 64 x 64 tiles with five 64-deep stages
// (each copy moves 8 rows of 128 bytes, whole cache lines of the row-major
// operands; 80 KiB of LDS, two workgroups per CU), K split as gemm_splits
// decides for Store / AddTo into partials.  Qwen-shaped layer at c = 16
// (cold weights): steps 302 / 311 / 338 -> 287 / 301 / 332 us at K = 3 / 5 / 7
// against the register-staged 128-row tiles; with 32-deep stages (half cache
// lines per copy) the K = 7 step was 354 us, and wider tiles (96 to 256
// columns, one workgroup per CU, more K splits) and six stages ran slower.
template <Epi EPI>
hipError_t launch_mid(GemvArgs& a, int num_cus, hipStream_t s) {
  return launch_ring<64, 64, 5, false, false, false, EPI, 64>(a, num_cus, s);
}

// Tile widths of the projections over more than 256 rows: 128 x 128 for
// q/k/v (the rotary epilogue spills on the wider tile), 128 x 256 for the
// rest.  The tile-major weight copies (launch_pack_proj_tiles) are packed in
// the load order of exactly these tiles.
template <Epi EPI>
constexpr int kManyRowsBN = EPI == Epi::QkvRope ? 128 : 256;

// Projections over more than 256 rows with the weights' tile-major copy and,
// for a plain operand, A written tile-major in 128-row groups by its producer
// (RMSNorm, attention merge, SiluMul epilogue): each copy instruction of the
// ring then reads one contiguous KiB of either operand.  Anything else is
// refused rather than run on a layout the kernel does not read.
template <Epi EPI, AMode MODE>
hipError_t launch_many_rows_packed(GemvArgs& a, int num_cus, hipStream_t s) {
  if (!a.pk_tiles || a.M <= 256 || a.ss_out) return hipErrorInvalidValue;
  if (a.y_group != 0 && (EPI != Epi::SiluMul || a.y_group != 128 || a.Nout % 32 != 0)) return hipErrorInvalidValue;
  if constexpr (MODE == AMode::Gather) {
    if constexpr (EPI == Epi::Store) {
      if (!a.part || a.x_group != 0) return hipErrorInvalidValue;
      return launch_ring<128, 256, 3, false, false, true, EPI, 32, true>(a, num_cus, s);
    }
    return hipErrorInvalidValue;
  } else {
    if (a.x_group != 128) return hipErrorInvalidValue;
    if constexpr (EPI == Epi::QkvRope || EPI == Epi::SiluMul)
      return launch_ring<128, kManyRowsBN<EPI>, EPI == Epi::QkvRope ? 4 : 3, false, true, true, EPI>(a, num_cus, s);
    else if constexpr (EPI == Epi::AddTo) {
      if (!a.part) return hipErrorInvalidValue;
      return launch_ring<128, 256, 3, false, true, true, EPI>(a, num_cus, s);
    }
    return hipErrorInvalidValue;
  }
}

template <Epi EPI, AMode MODE>
hipError_t launch_cfg(GemvArgs& a, int num_cus, hipStream_t s) {
  if constexpr (EPI != Epi::Argmax) {
    if (a.pk_tiles || a.x_group || a.y_group) return launch_many_rows_packed<EPI, MODE>(a, num_cus, s);
  }
  // Many rows (more than two 128-row tiles) on a plain operand: the LDS-DMA
  // ring on row-major W -- 128 x 256 tiles (K split when the caller takes
  // partials), 128 x 128 for q/k/v (the rotary epilogue spills on the wider
  // tile).  At 672 rows it ran the o / down / gate-up / q-k-v projections
  // 7-18% faster than the register-staged tiles.
  if constexpr (MODE == AMode::Plain && EPI != Epi::Argmax) {
    if (a.M > 256 && !a.ss_out) {
      if constexpr (EPI == Epi::QkvRope)
        return launch_ring<128, 128, 4, false, false, false, EPI>(a, num_cus, s);
      else if constexpr (EPI == Epi::SiluMul)
        return launch_ring<128, 256, 3, false, false, false, EPI>(a, num_cus, s);
      else if (a.part)
        return launch_ring<128, 256, 3, false, false, false, EPI>(a, num_cus, s);
    }
  }
  if constexpr (MODE == AMode::Plain && EPI != Epi::Argmax) {
    if (a.M > 16 && a.M <= 256 && !a.ss_out && a.K % 64 == 0 &&
        (EPI == Epi::QkvRope || EPI == Epi::SiluMul || a.part))
      return launch_mid<EPI>(a, num_cus, s);
  }
  // The fc input gathered on the fly ([embed[id] ; h] rows) into partials:
  // the same rings as the plain residual projections, each stage taken from
  // one half.
  if constexpr (MODE == AMode::Gather && EPI == Epi::Store) {
    if (a.part && !a.ss_out) {
      if (a.M > 256 && (a.K / 2) % 32 == 0)
        return launch_ring<128, 256, 3, false, false, false, EPI, 32, true>(a, num_cus, s);
      if (a.M > 16 && (a.K / 2) % 64 == 0)
        return launch_ring<64, 64, 5, false, false, false, EPI, 64, true>(a, num_cus, s);
    }
  }
  TileCfg t = pick_tile(a.M, a.Nout, EPI, num_cus);
  // Store / AddTo into split partials: 128 x 128 tiles, K split to fill the CUs
  if ((EPI == Epi::Store || EPI == Epi::AddTo) && a.part && !a.ss_out &&
      tiles_of(t, a.M, a.Nout, EPI) < 2 * num_cus)
    t = kMedium;
  if (t.bn == 256) {
    // (never chosen for q/k/v, whose epilogue does not fit this tile's registers)
    if constexpr (EPI == Epi::QkvRope) return hipErrorInvalidValue;
    else return launch_t<128, 256, 32, 2, 2, EPI, MODE>(a, num_cus, s);
  }
  if (t.bn == 128) return launch_t<128, 128, 64, 2, 2, EPI, MODE>(a, num_cus, s);
  return launch_t<128, 64, 64, 2, 2, EPI, MODE>(a, num_cus, s);
}

// dst[((g * (K / 32) + kt) * 256 + r) * 32 + c] = W[g * 256 + r][kt * 32 + c],
// rows past Nout zero; one thread per 16-byte chunk
__global__ void pack_tiles_kernel(const bf16_t* __restrict__ w, bf16_t* __restrict__ dst, int Nout, int K,
                                  int64_t chunks) {
  const int nk = K / 32;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < chunks;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(i & 3);
    const int64_t rest = i >> 2;
    const int r = static_cast<int>(rest % kTileGroup);
    const int64_t rest2 = rest / kTileGroup;
    const int kt = static_cast<int>(rest2 % nk);
    const int64_t row = (rest2 / nk) * kTileGroup + r;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < Nout) v = load16(w + row * K + kt * 32 + c * 8);
    store16(dst + i * 8, v);
  }
}

// Tile-major copy of a projection in its ring tiles' load order: packed row
// R is row R % BN of N tile R / BN (b_ptr, which clamps past the last W row),
// rows past the last tile zero; layout and thread mapping as pack_tiles_kernel
template <Epi EPI, int BN>
__global__ void pack_proj_tiles_kernel(GemvArgs a, bf16_t* __restrict__ dst, int rows, int64_t chunks) {
  const int nk = a.K / 32;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < chunks;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(i & 3);
    const int64_t rest = i >> 2;
    const int r = static_cast<int>(rest % kTileGroup);
    const int64_t rest2 = rest / kTileGroup;
    const int kt = static_cast<int>(rest2 % nk);
    const int64_t row = (rest2 / nk) * kTileGroup + r;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < rows)
      v = load16(b_ptr<EPI, BN, BN / 2>(a, static_cast<int>(row / BN), static_cast<int>(row % BN)) + kt * 32 + c * 8);
    store16(dst + i * 8, v);
  }
}

// rows the ring's N tiles load over > 256 rows (whole tiles)
int many_rows_tile_rows(Epi epi, int Nout) {
  const int bn = epi == Epi::QkvRope ? kManyRowsBN<Epi::QkvRope> : kManyRowsBN<Epi::Store>;
  const int cols = epi == Epi::SiluMul ? bn / 2 : bn;
  return (Nout + cols - 1) / cols * bn;
}

template <Epi EPI>
hipError_t pack_proj_t(const GemvArgs& a, void* dst, hipStream_t s) {
  const int rows = many_rows_tile_rows(EPI, a.Nout);
  const int64_t chunks = static_cast<int64_t>(proj_tile_bytes(EPI, a.Nout, a.K) / 16);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 16384);
  hipLaunchKernelGGL((pack_proj_tiles_kernel<EPI, kManyRowsBN<EPI>>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                     0, s, a, static_cast<bf16_t*>(dst), rows, chunks);
  return hipGetLastError();
}

}  // namespace

size_t proj_tile_bytes(Epi epi, int Nout, int K) {
  const int rows = many_rows_tile_rows(epi, Nout);
  return static_cast<size_t>((rows + kTileGroup - 1) / kTileGroup) * kTileGroup * K * 2;
}

hipError_t launch_pack_proj_tiles(Epi epi, const GemvArgs& a, void* dst, hipStream_t s) {
  if (!dst || !a.w_a || !a.w_b || !a.w_c || a.Nout <= 0 || a.K <= 0 || a.K % 32 != 0) return hipErrorInvalidValue;
  switch (epi) {
    case Epi::Store:
    case Epi::AddTo: return pack_proj_t<Epi::AddTo>(a, dst, s);
    case Epi::SiluMul: return pack_proj_t<Epi::SiluMul>(a, dst, s);
    case Epi::QkvRope:
      if (a.rope.d != 16 && a.rope.d != 32 && a.rope.d != 64 && a.rope.d != 128) return hipErrorInvalidValue;
      return pack_proj_t<Epi::QkvRope>(a, dst, s);
    default: return hipErrorInvalidValue;
  }
}

size_t packed_tile_bytes(int Nout, int K) {
  return static_cast<size_t>((Nout + kTileGroup - 1) / kTileGroup) * kTileGroup * K * 2;
}

hipError_t launch_pack_tiles(const void* w, int Nout, int K, void* dst, hipStream_t s) {
  if (!w || !dst || Nout <= 0 || K <= 0 || K % 32 != 0) return hipErrorInvalidValue;
  const int64_t chunks = static_cast<int64_t>(packed_tile_bytes(Nout, K) / 16);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 16384);
  hipLaunchKernelGGL(pack_tiles_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(w), static_cast<bf16_t*>(dst), Nout, K, chunks);
  return hipGetLastError();
}

int gemm_parts(int M, int Nout, int num_cus) {
  const TileCfg t = pick_tile(M, Nout, Epi::Argmax, num_cus);
  return (Nout + t.bn - 1) / t.bn;
}

hipError_t launch_gemm(GemvArgs& a, Epi epi, int num_cus, hipStream_t s) {
  if (epi == Epi::QkvRope && !a.rope.table) return hipErrorInvalidValue;
  if (a.amode == AMode::Gather) {
    if (epi == Epi::Store) return launch_cfg<Epi::Store, AMode::Gather>(a, num_cus, s);
    return hipErrorInvalidValue;
  }
  if (a.amode != AMode::Plain) return hipErrorInvalidValue;
  switch (epi) {
    case Epi::Store: return launch_cfg<Epi::Store, AMode::Plain>(a, num_cus, s);
    case Epi::AddTo: return launch_cfg<Epi::AddTo, AMode::Plain>(a, num_cus, s);
    case Epi::SiluMul: return launch_cfg<Epi::SiluMul, AMode::Plain>(a, num_cus, s);
    case Epi::QkvRope: return launch_cfg<Epi::QkvRope, AMode::Plain>(a, num_cus, s);
    case Epi::Argmax:
      // with the tile-major copy: the LDS-DMA ring, 128 x 256 tiles (fragment
      // prefetch once several M tiles share each W tile)
      // (tile-major activations too when the producer wrote them so)
      if (a.pk_tiles) {
        if (a.x_group == 128) {
          if (a.M > 128) return launch_ring<128, 256, 3, true, true, true, Epi::Argmax>(a, num_cus, s);
          return launch_ring<128, 256, 3, false, true, true, Epi::Argmax>(a, num_cus, s);
        }
        if (a.x_group != 0) return hipErrorInvalidValue;
        if (a.M > 128) return launch_ring<128, 256, 3, true, false, true, Epi::Argmax>(a, num_cus, s);
        return launch_ring<128, 256, 3, false, false, true, Epi::Argmax>(a, num_cus, s);
      }
      if (a.x_group != 0) return hipErrorInvalidValue;
      return launch_cfg<Epi::Argmax, AMode::Plain>(a, num_cus, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pe
