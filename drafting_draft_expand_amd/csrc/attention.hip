// Paged grouped-query attention of the draft rows, split over the KV range.
//
// Every non-rejected draft row at position p attends to positions 0..p of its
// own sequence (the cached context plus the rows this pass just wrote), with
// q head h reading kv head h / (n_q / n_kv).  The causal mask compares
// POSITIONS, not row indices: MASK rows sit at positions after the bonus row
// while rejected rows keep older positions and are skipped entirely.
//
// Grid (split, kv head, sequence).  A workgroup owns all query heads of one
// kv-head group for every row of its sequence, and one contiguous slice of the
// sequence's key positions; 64-key K/V tiles are gathered page by page into LDS
// (fp32) and scored against a 64-query tile kept in LDS, with an fp32 online
// softmax.  Each (row, head, split) leaves (acc[d], max, sum) in the workspace
// and a second kernel merges the splits with their log-sum-exp weights and
// stores the attention output as the next projection's operand.
#include "common.h"

namespace pe {
namespace {

constexpr int QT = 64;  // queries per tile
constexpr int KT = 64;  // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  __shared__ float qs[QT][D + 1];
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[KT][D + 1];
  __shared__ float sc[QT][KT + 1];
  __shared__ int qpos[QT];
  const int tid = threadIdx.x;
  const int sp = blockIdx.x, g = blockIdx.y, i = blockIdx.z;
  const int grp = a.n_q / a.n_kv;
  const int r0 = a.cu_draft[i], r1 = a.cu_draft[i + 1];
  const int kvlen = a.kv_lens[i];
  const int chunk = ((kvlen + a.splits - 1) / a.splits + 15) / 16 * 16;
  const int kb = sp * chunk;
  const int ke = min(kvlen, kb + chunk);
  const int nqry = (r1 - r0) * grp;
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  const T* qin = static_cast<const T*>(a.q);
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
  constexpr int DP = D / 4;  // dims per thread in the PV update

  for (int qt0 = 0; qt0 < nqry; qt0 += QT) {
    for (int e = tid; e < QT * D; e += 256) {
      const int qi = e / D, dd = e - qi * D;
      const int q = qt0 + qi;
      float v = 0.f;
      if (q < nqry) {
        const int row = r0 + q / grp, h = g * grp + q % grp;
        v = Elem<T>::to_f32(qin[(static_cast<int64_t>(row) * a.n_q + h) * D + dd]) * scale;
      }
      qs[qi][dd] = v;
    }
    if (tid < QT) {
      const int q = qt0 + tid;
      int p = -1;  // -1: inactive query (past the end or rejected row)
      if (q < nqry) {
        const int row = r0 + q / grp;
        if (!a.rejected[row]) p = a.pos[row];
      }
      qpos[tid] = p;
    }
    const int qi = tid >> 2, part = tid & 3;
    float m_run = -INFINITY, l_run = 0.f;
    float acc[DP];
#pragma unroll
    for (int x = 0; x < DP; ++x) acc[x] = 0.f;
    __syncthreads();

    for (int kt0 = kb; kt0 < ke; kt0 += KT) {
      for (int e = tid; e < KT * D; e += 256) {
        const int kk = e / D, dd = e - kk * D;
        const int p = kt0 + kk;
        float kv = 0.f, vv = 0.f;
        if (p < ke) {
          const int64_t blk = bt[p / a.block_size];
          const int64_t base = ((blk * a.n_kv + g) * a.block_size + p % a.block_size) * D + dd;
          kv = Elem<T>::to_f32(kc[base]);
          vv = Elem<T>::to_f32(vc[base]);
        }
        ks[kk][dd] = kv;
        vs[kk][dd] = vv;
      }
      __syncthreads();
      {
        const int q2 = tid & 63;
        const int k0 = (tid >> 6) * 16;
        const int qp = qpos[q2];
        for (int kk = 0; kk < 16; ++kk) {
          const int key = k0 + kk;
          const int p = kt0 + key;
          float s = -INFINITY;
          if (p < ke && p <= qp) {
            s = 0.f;
#pragma unroll 16
            for (int dd = 0; dd < D; ++dd) s = fmaf(qs[q2][dd], ks[key][dd], s);
          }
          sc[q2][key] = s;
        }
      }
      __syncthreads();
      {
        float mx = -INFINITY;
        for (int kk = 0; kk < KT; ++kk) mx = fmaxf(mx, sc[qi][kk]);
        const float mnew = fmaxf(m_run, mx);
        if (mnew != -INFINITY) {
          const float corr = m_run == -INFINITY ? 0.f : expf(m_run - mnew);
          l_run *= corr;
#pragma unroll
          for (int x = 0; x < DP; ++x) acc[x] *= corr;
          for (int kk = 0; kk < KT; ++kk) {
            const float s = sc[qi][kk];
            if (s == -INFINITY) continue;
            const float pr = expf(s - mnew);
            l_run += pr;
#pragma unroll
            for (int x = 0; x < DP; ++x) acc[x] = fmaf(pr, vs[kk][part * DP + x], acc[x]);
          }
          m_run = mnew;
        }
      }
      __syncthreads();
    }

    const int q = qt0 + qi;
    if (q < nqry) {
      const int row = r0 + q / grp, h = g * grp + q % grp;
      float* o = a.partial + ((static_cast<int64_t>(row) * a.n_q + h) * a.splits + sp) * (D + 2);
#pragma unroll
      for (int x = 0; x < DP; ++x) o[part * DP + x] = acc[x];
      if (part == 0) {
        o[D] = m_run;
        o[D + 1] = l_run;
      }
    }
    __syncthreads();
  }
}

// bf16, head_dim 64/128: the same split-KV attention on MFMA.
//
// A workgroup of 8 waves owns up to 128 queries (16 per wave) of one
// (sequence, kv head, split).  Per 64-key tile the waves share K and V in
// LDS.  Scores are formed transposed, S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (keys are the A rows, the wave's queries the B
// columns), so each lane owns one query column: the online-softmax row
// statistics need only the 4 lanes that share that column, and the
// probabilities are already in the B-operand layout of O^T += V^T P^T.  In
// that product the MFMA's 32 k-slots of each 32-key half enumerate keys
// 4j..4j+3 and 16+4j..16+4j+3 for lane group j, the order in which the score
// tiles hold them.  K and V both stay row-major in
// double-buffered LDS and the V^T operand of O^T += V^T P^T is formed by the
// transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i % 4 of the 64-bit words read by lanes 4q + i / 4,
// q = 0..3.  Lane 4q + c of group j therefore reads the four dims
// 16 t + 4c .. 16 t + 4c + 3 of key 4j + q (and of key 16 + 4j + q for the
// second word), which hands lane i of group j exactly the dim 16 t + i of
// keys 4j..4j+3 and 16+4j..16+4j+3 -- the key order of the score tiles.  Rows
// are padded by 32 bytes so the 16-row fragment reads and the transposing
// reads spread over all banks.  One barrier per 64-key tile: tile t + 1 is
// written to the other buffer while tile t is consumed.
template <int D, int DEPTH, int OCC, bool LP>
__global__ __launch_bounds__(512, OCC) void attn_mfma_kernel(AttnArgs a) {
  constexpr int KT = 64;
  constexpr int RP = D + 16;   // padded K / V row (elements)
  constexpr int DT = D / 16;   // O^T tiles
  constexpr int KK = D / 32;   // k-steps of S^T
  constexpr int PER = KT * D / 8 / 512;  // 16-byte K (and V) pieces per thread per tile
  static_assert(PER >= 1, "tile too small for the workgroup");
  // LP: the split's page numbers sit in LDS (the host checked they fit), so
  // K/V addresses do not wait on a block-table load
  constexpr int MAXB = LP ? kAttnMaxPages : 1;
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][KT * RP];
  __shared__ __attribute__((aligned(16))) bf16_t vs[2][KT * RP];
  __shared__ int32_t pages[MAXB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, j = lane >> 4;
  const int sp = blockIdx.x, g = blockIdx.y, i = blockIdx.z;
  const int grp = a.n_q / a.n_kv;
  const int r0 = a.cu_draft[i], r1 = a.cu_draft[i + 1];
  const int kvlen = a.kv_lens[i];
  const int chunk = ((kvlen + a.splits - 1) / a.splits + KT - 1) / KT * KT;
  const int kb = sp * chunk;
  const int ke = min(kvlen, kb + chunk);
  const int ntiles = ke > kb ? (ke - kb + KT - 1) / KT : 0;
  const int nqry = (r1 - r0) * grp;
  const float sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));  // scale * log2(e)
  const bf16_t* qin = static_cast<const bf16_t*>(a.q);
  const bf16_t* kc = static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vc = static_cast<const bf16_t*>(a.v_cache);
  const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int BS = 16;  // KV page size (the only one the library accepts)
  const int pg0 = kb / BS;
  const int npg = ke > kb ? (ke - 1) / BS - pg0 + 1 : 0;
  if (LP)
    for (int q = tid; q < min(npg, MAXB); q += 512) pages[q] = bt[pg0 + q];
  __syncthreads();

  // DEPTH tiles in flight in registers beyond the one in LDS; tile u waits in
  // register set u % DEPTH and is consumed from LDS buffer u % 2
  static_assert(DEPTH >= 2 && DEPTH <= 4, "2..4 tiles in flight");
  constexpr int U = DEPTH % 2 == 0 ? DEPTH : 2 * DEPTH;
  u32x4 kr[DEPTH][PER], vr[DEPTH][PER];
  // Requests are unconditional (positions past the split's end are clamped to
  // its last key, whose values are finite and whose probability is zero), so
  // every lane issues the same loads and the compiler's counters of
  // outstanding loads stay exact: staging tile t + 1 waits only for it.
  auto fetch = [&](int t, auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int pp = 0; pp < PER; ++pp) {
      const int piece = tid + 512 * pp;
      const int key = piece / (D / 8), c8 = piece % (D / 8);
      const int p = min(kb + t * KT + key, ke - 1);
      const int64_t blk = LP ? pages[p / BS - pg0] : bt[p / BS];
      const int64_t off = ((blk * a.n_kv + g) * BS + p % BS) * D + c8 * 8;
      kr[set][pp] = load16(kc + off);
      vr[set][pp] = load16(vc + off);
    }
  };
  auto stash = [&](auto buf_c, auto set_c) {
    constexpr int buf = decltype(buf_c)::value, set = decltype(set_c)::value;
#pragma unroll
    for (int pp = 0; pp < PER; ++pp) {
      const int piece = tid + 512 * pp;
      const int key = piece / (D / 8), c8 = piece % (D / 8);
      store16(&ks[buf][key * RP + c8 * 8], kr[set][pp]);
      store16(&vs[buf][key * RP + c8 * 8], vr[set][pp]);
    }
  };

  for (int qb = 0; qb < nqry; qb += 128) {
    const int qn = qb + wave * 16 + (lane & 15);
    const int row = r0 + qn / grp;
    const int h = g * grp + qn % grp;
    const bool active = qn < nqry && !a.rejected[row];
    const int qpos = active ? a.pos[row] : -1;
    // smallest causal bound among this wave's active queries
    int wave_qmin = active ? qpos : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wave_qmin = min(wave_qmin, __shfl_xor(wave_qmin, off, 64));
    // a wave whose 16 queries are all past the end or on rejected rows skips
    // the products (it still stages its share of every K/V tile)
    const bool wave_live = __builtin_amdgcn_readfirstlane(wave_qmin) != 0x7fffffff;
    u32x4 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = active ? load16(qin + (static_cast<int64_t>(row) * a.n_q + h) * D + 32 * kk + 8 * j) : zero;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int t, auto buf_c) {
      constexpr int buf = decltype(buf_c)::value;
      const int kt0 = kb + t * KT;
      f32x4 st[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // d-slices outer, key tiles inner: consecutive MFMAs are independent
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const u32x4 af =
              *reinterpret_cast<const u32x4*>(&ks[buf][(mt * 16 + (lane & 15)) * RP + 32 * kk + 8 * j]);
          st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                           __builtin_bit_cast(bf16x8, qf[kk]), st[mt], 0, 0, 0);
        }
      // online softmax in base 2 with the 1/sqrt(d) scale folded into one FMA:
      // p = 2^(s * sl2 - m), m the running maximum of s * sl2.  A tile that
      // lies wholly inside every query's causal range of this wave (the common
      // case) skips the per-key masks.
      const bool full = kt0 + KT <= ke && kt0 + KT - 1 <= wave_qmin;
      float sv[16];
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sv[mt * 4 + q] = st[mt][q];
            mx = fmaxf(mx, st[mt][q]);
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int p = kt0 + mt * 16 + 4 * j + q;
            const float sc = (p < ke && p <= qpos) ? st[mt][q] : -INFINITY;
            sv[mt * 4 + q] = sc;
            mx = fmaxf(mx, sc);
          }
      }
      mx = xor32_max(xor16_max(mx));
      const float m_new = fmaxf(m_run, mx * sl2);
      // all keys so far masked: keep the sums at zero (m_new = -inf)
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
      float rs = 0.f;
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[2 * e], sl2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[2 * e + 1], sl2, -m_use));
        rs += p0 + p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      rs = xor32_sum(xor16_sum(rs));
      l_run = l_run * corr + rs;
      m_run = m_new;
      // transposing-read address of this lane: key 4j + (lane % 16) / 4, dims
      // 4 (lane % 4) .. + 3 of each 16-dim tile
      const bf16_t* vb = &vs[buf][(4 * j + ((lane & 15) >> 2)) * RP + 4 * (lane & 3)];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 pb = {pk[4 * hf], pk[4 * hf + 1], pk[4 * hf + 2], pk[4 * hf + 3]};
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) {
          if (hf == 0) o[t2] *= corr;
          const bf16_t* src = vb + (hf * 32) * RP + t2 * 16;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(src));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(src + 16 * RP));
          const u32x4 af = {__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                            __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
          o[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                          __builtin_bit_cast(bf16x8, pb), o[t2], 0, 0, 0);
        }
      }
    };

    // prologue: tiles 0 .. DEPTH - 1 requested, tile 0 published in buffer 0,
    // tile DEPTH requested into the freed register set
    if (ntiles > 0) {
      static_for<DEPTH>([&](auto s_c) { fetch(min(static_cast<int>(decltype(s_c)::value), ntiles - 1), s_c); });
      using Z = std::integral_constant<int, 0>;
      stash(Z{}, Z{});
      fetch(min(DEPTH, ntiles - 1), Z{});
    }
    __syncthreads();
    // tile t: consume its buffer, publish tile t + 1 in the other buffer,
    // request tile t + 1 + DEPTH into the register set tile t + 1 freed
    for (int t0 = 0; t0 < ntiles; t0 += U) {
      static_for<U>([&](auto j_c) {
        constexpr int jj = decltype(j_c)::value;
        const int t = t0 + jj;
        if (t < ntiles) {
          if (wave_live) compute(t, std::integral_constant<int, jj & 1>{});
          using Nb = std::integral_constant<int, (jj + 1) & 1>;
          using Ns = std::integral_constant<int, (jj + 1) % DEPTH>;
          // past the last tile these publish / request clamped, unused data
          stash(Nb{}, Ns{});
          fetch(min(t + 1 + DEPTH, ntiles - 1), Ns{});
          __syncthreads();
        }
      });
    }
    if (qn < nqry && !a.rejected[row]) {
      float* out = a.partial + ((static_cast<int64_t>(row) * a.n_q + h) * a.splits + sp) * (D + 2);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) out[t * 16 + 4 * j + q] = o[t][q];
      if (j == 0) {
        // row statistics in natural-log units for the combine step
        out[D] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
        out[D + 1] = l_run;
      }
    }
    __syncthreads();
  }
}

// bf16, 64- or 128-dim heads, a split's page numbers in LDS: the same
// products with K and V copied straight into a ring of ST LDS stages
// (global_load_lds, no register staging), so the copies of later tiles run
// while the waves compute instead of between their products.  A stage holds
// the tile's 64 K rows then its 64 V rows, each as D / 64 planes of 64 dims
// (128 bytes a row, unpadded), 16-byte chunk c of key row r of a plane at
// slot c ^ (r & 7): the score-fragment reads (16 rows x 4 chunks) and the
// transposing V reads both spread over the banks, and a 128-dim tile is read
// as two 64-dim ones.  Wave w copies keys 8w..8w+7 of each plane of K and of
// V (one KiB each; eight keys never straddle a 16-token page).  Step t waits
// until its own copies of stage t have landed (ST-2 stages still in flight),
// meets the other waves, requests tile t+ST-1 into the slot step t-1 used,
// then computes.  Two stages (ST = 2) make it a double buffer: every copy of
// tile t has landed before the barrier of step t.  64-dim heads with three
// stages and 128-dim heads with two fit two workgroups per CU.
template <int D, int ST>
__global__ __launch_bounds__(512, D == 64 || ST == 2 ? 4 : 2) void attn_ring_kernel(AttnArgs a) {
  constexpr int KT = 64, PL = D / 64;  // keys per tile, 64-dim planes
  constexpr int DT = D / 16, KK = D / 32;
  constexpr int SK = KT * D;  // elements of one K (or V) tile
  constexpr int SP = KT * 64;  // elements of one plane of a tile
  constexpr int BS = 16;       // KV page size (the only one the library accepts)
  static_assert(D == 64 || D == 128, "64- or 128-dim heads");
  static_assert(ST >= 2 && ST <= 4, "two to four ring stages");
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) bf16_t R0[2 * SK];
  __shared__ __attribute__((aligned(16))) bf16_t R1[2 * SK];
  __shared__ __attribute__((aligned(16))) bf16_t R2[ST > 2 ? 2 * SK : 8];
  __shared__ __attribute__((aligned(16))) bf16_t R3[ST > 3 ? 2 * SK : 8];
  __shared__ int32_t pages[kAttnMaxPages];
  auto ring = [&](auto s_c) __attribute__((always_inline)) -> bf16_t* {
    constexpr int S = decltype(s_c)::value % ST;
    if constexpr (S == 0) return R0;
    else if constexpr (S == 1) return R1;
    else if constexpr (S == 2) return R2;
    else return R3;
  };
  const int tid = threadIdx.x, lane = tid & 63, j = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sp = blockIdx.x, g = blockIdx.y;
  // Longest KV ranges first: the workgroups of launch slot z take the
  // sequence of rank z by decreasing KV length (ties by index), so the
  // longest splits start at once and the short ones fill in behind them
  // instead of a long one starting last (one sequence, or more than 512:
  // launch order).
  __shared__ int seq_sel;
  int i = blockIdx.z;
  if (a.c > 1 && a.c <= 512) {
    if (tid < a.c) {
      const int mine = a.kv_lens[tid];
      int rank = 0;
      for (int o = 0; o < a.c; ++o) {
        const int other = a.kv_lens[o];
        rank += other > mine || (other == mine && o < tid);
      }
      // launch slot z takes rank z, or with `fold` the second half of the
      // slots the remaining ranks from the shortest up
      const int z = blockIdx.z, h = (a.c + 1) / 2;
      const int want = a.fold && z >= h ? a.c - 1 - (z - h) : z;
      if (rank == want) seq_sel = tid;
    }
    __syncthreads();
    i = __builtin_amdgcn_readfirstlane(seq_sel);
  }
  const int grp = a.n_q / a.n_kv;
  const int r0 = a.cu_draft[i], r1 = a.cu_draft[i + 1];
  const int kvlen = a.kv_lens[i];
  const int chunk = ((kvlen + a.splits - 1) / a.splits + KT - 1) / KT * KT;
  const int kb = sp * chunk;
  const int ke = min(kvlen, kb + chunk);
  const int ntiles = ke > kb ? (ke - kb + KT - 1) / KT : 0;
  const int nqry = (r1 - r0) * grp;
  const float sl2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));  // scale * log2(e)
  const bf16_t* qin = static_cast<const bf16_t*>(a.q);
  const bf16_t* kc = static_cast<const bf16_t*>(a.k_cache);
  const bf16_t* vc = static_cast<const bf16_t*>(a.v_cache);
  const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // This lane's query of block qb: its row (clamped into the sequence for the
  // loads), head, rejected flag, position and fragments, all loaded without a
  // branch so that they are in flight together; those of the first block go
  // out before the page list is fetched.
  struct Query {
    int qn, row, h;
    bool rej;
    int pos;
    u32x4 qf[KK];
  };
  auto load_query = [&](int qb) __attribute__((always_inline)) {
    Query q;
    q.qn = qb + wave * 16 + (lane & 15);
    q.row = min(r0 + q.qn / grp, r1 - 1);
    q.h = g * grp + q.qn % grp;
    q.rej = a.rejected[q.row] != 0;
    q.pos = a.pos[q.row];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) q.qf[kk] = load16(qin + (static_cast<int64_t>(q.row) * a.n_q + q.h) * D + 32 * kk + 8 * j);
    return q;
  };
  Query qnext = load_query(0);
  const int pg0 = kb / BS;
  const int npg = ke > kb ? (ke - 1) / BS - pg0 + 1 : 0;
  for (int q = tid; q < min(npg, kAttnMaxPages); q += 512) pages[q] = bt[pg0 + q];
  __syncthreads();

  // this lane's copy: key 8 wave + lane / 8 of the tile, slot lane % 8, which
  // holds global chunk (lane % 8) ^ (key & 7).  A wave's eight keys lie in
  // one 16-token page (also after clamping to the split's last key), so the
  // page and its base address are the same for the whole wave.
  const int cgc = (lane & 7) ^ ((lane >> 3) & 7);
  auto request = [&](int t, auto s_c) __attribute__((always_inline)) {
    bf16_t* st = ring(s_c);
    const int p0 = kb + min(t, ntiles - 1) * KT + wave * 8;  // the wave's first key
    const int page = __builtin_amdgcn_readfirstlane(pages[min(p0, ke - 1) / BS - pg0]);
    const int64_t base = (static_cast<int64_t>(page) * a.n_kv + g) * BS * D;
    // clamped to the split's last key: finite values whose probability is zero
    const int p = min(p0 + (lane >> 3), ke - 1);
    const int off = (p % BS) * D + cgc * 8;
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
      dma16<true>(kc + base + off + pl * 64, st + pl * SP + wave * 8 * 64);
      dma16<true>(vc + base + off + pl * 64, st + SK + pl * SP + wave * 8 * 64);
    }
  };
  constexpr int kWait = waitcnt_vm_lgkm0((ST - 2) * 2 * PL);

  for (int qb = 0; qb < nqry; qb += 128) {
    const Query cur = qnext;
    const int qn = cur.qn, row = cur.row, h = cur.h;
    const bool active = qn < nqry && !cur.rej;
    const int qpos = active ? cur.pos : -1;
    int wave_qmin = active ? qpos : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wave_qmin = min(wave_qmin, __shfl_xor(wave_qmin, off, 64));
    const bool wave_live = __builtin_amdgcn_readfirstlane(wave_qmin) != 0x7fffffff;
    u32x4 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = active ? cur.qf[kk] : zero;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int t, auto s_c) __attribute__((always_inline)) {
      const bf16_t* ks = ring(s_c);
      const bf16_t* vs = ks + SK;
      const int kt0 = kb + t * KT;
      f32x4 st[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int r = mt * 16 + (lane & 15);
          const bf16_t* kp = ks + (kk >> 1) * SP + r * 64;  // plane kk / 2, its chunk 4 (kk % 2) + j
          const u32x4 af = *reinterpret_cast<const u32x4*>(&kp[((4 * (kk & 1) + j) ^ (r & 7)) << 3]);
          st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                           __builtin_bit_cast(bf16x8, qf[kk]), st[mt], 0, 0, 0);
        }
      const bool full = kt0 + KT <= ke && kt0 + KT - 1 <= wave_qmin;
      float sv[16];
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sv[mt * 4 + q] = st[mt][q];
            mx = fmaxf(mx, st[mt][q]);
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int p = kt0 + mt * 16 + 4 * j + q;
            const float sc = (p < ke && p <= qpos) ? st[mt][q] : -INFINITY;
            sv[mt * 4 + q] = sc;
            mx = fmaxf(mx, sc);
          }
      }
      mx = xor32_max(xor16_max(mx));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      // the running sums need rescaling only where the maximum rose (elsewhere
      // the factor is exactly 1): skipped when it rose nowhere in the wave
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= corr;
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) o[t2] *= corr;
      }
      float rs = 0.f;
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[2 * e], sl2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[2 * e + 1], sl2, -m_use));
        rs += p0 + p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      rs = xor32_sum(xor16_sum(rs));
      l_run += rs;
      m_run = m_new;
      // transposing V reads: lane 4q + c of group j reads dims 16 t + 4 c ..
      // + 3 of key 4 j + q (+ 16 for the second word, + 32 for the second
      // half), i.e. chunk 2 (t % 4) + c / 2, element 4 (c % 2) of that key
      // row in plane t / 4
      const int kq = 4 * j + ((lane & 15) >> 2);
      const int cq = lane & 3;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 pb = {pk[4 * hf], pk[4 * hf + 1], pk[4 * hf + 2], pk[4 * hf + 3]};
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) {
          const int ra = kq + hf * 32, rb = ra + 16;
          const int cc = 2 * (t2 & 3) + (cq >> 1), e4 = 4 * (cq & 1);
          const bf16_t* vp = vs + (t2 >> 2) * SP;
          const bf16_t* sa = vp + ra * 64 + ((cc ^ (ra & 7)) << 3) + e4;
          const bf16_t* sb = vp + rb * 64 + ((cc ^ (rb & 7)) << 3) + e4;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(sa));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(sb));
          const u32x4 af = {__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                            __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
          o[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                          __builtin_bit_cast(bf16x8, pb), o[t2], 0, 0, 0);
        }
      }
    };
    auto step = [&](int t, auto s_c) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value;
      __builtin_amdgcn_s_waitcnt(kWait);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      request(t + ST - 1, std::integral_constant<int, (S + ST - 1) % ST>{});
      if (wave_live) compute(t, s_c);
    };

    if (ntiles > 0) {
      static_for<ST - 1>([&](auto s_c) { request(decltype(s_c)::value, s_c); });
      // the query fragments and the first stages: one wait, so no product in
      // the loop waits on global memory the compiler tracks
      __builtin_amdgcn_s_waitcnt(0);
      int t = 0;
      for (; t + ST <= ntiles; t += ST) static_for<ST>([&](auto s_c) { step(t + decltype(s_c)::value, s_c); });
      static_for<ST - 1>([&](auto s_c) {
        if (t + decltype(s_c)::value < ntiles) step(t + decltype(s_c)::value, s_c);
      });
      // every copy (clamped repeats included) has landed before the ring is
      // reused or the workgroup ends
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    if (active) {
      float* out = a.partial + ((static_cast<int64_t>(row) * a.n_q + h) * a.splits + sp) * (D + 2);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) out[t * 16 + 4 * j + q] = o[t][q];
      if (j == 0) {
        out[D] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
        out[D + 1] = l_run;
      }
    }
    if (qb + 128 < nqry) qnext = load_query(qb + 128);
  }
}

// out[row, h, :] = sum_s acc_s * e^{m_s - M} / sum_s l_s * e^{m_s - M} (zero
// for a rejected row); four waves per workgroup, HPW heads per wave.  Every
// load is issued before the first use: lane s reads the statistics of split
// s, and every lane reads its output dims (lane, lane + 64) of all splits,
// splits past S clamped to the last one and weighted 0, so the kernel waits
// for memory once.
template <typename T, int D, int MAXS, int HPW>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int DV = (D + 63) / 64;  // output dims per lane
  const int row = blockIdx.x, lane = threadIdx.x & 63;
  const int h0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * HPW;  // this wave's first head
  const int S = a.splits;                                      // 1 <= S <= MAXS
  const bool rejected = a.rejected[row];
  const int sl = min(lane, S - 1);
  // (a rejected row's partials were never written: they are read with the
  // rest, so no load waits for the flag, and discarded)
  auto load_head = [&](int h, float& m_l, float& l_l, float (&v)[DV][MAXS]) __attribute__((always_inline)) {
    const float* p = a.partial + (static_cast<int64_t>(row) * a.n_q + h) * S * (D + 2);
    m_l = p[sl * (D + 2) + D];
    l_l = p[sl * (D + 2) + D + 1];
#pragma unroll
    for (int z = 0; z < MAXS; ++z) {
      const int zc = min(z, S - 1);
#pragma unroll
      for (int e = 0; e < DV; ++e) v[e][z] = p[zc * (D + 2) + min(lane + 64 * e, D - 1)];
    }
  };
  // element h D + e of the row: row-major, or tile-major in groups of
  // out_group rows (32-element pieces of one row contiguous)
  const int G = a.out_group;
  T* out = static_cast<T*>(a.out);
  auto merge_store = [&](int h, float m_l, float l_l, const float (&v)[DV][MAXS]) __attribute__((always_inline)) {
    auto out_at = [&](int e) -> int64_t {
      const int64_t k = static_cast<int64_t>(h) * D + e;
      if (G == 0) return static_cast<int64_t>(row) * a.n_q * D + k;
      return (static_cast<int64_t>(row / G) * (a.n_q * D / 32) + k / 32) * G * 32 + (row % G) * 32 + (k & 31);
    };
    const float ms = lane < S ? m_l : -INFINITY;
    const float M = wave_max(ms);
    const float w = ms == -INFINITY ? 0.f : expf(ms - M);
    const float den = wave_sum(lane < S ? w * l_l : 0.f);
    float num[DV];
#pragma unroll
    for (int e = 0; e < DV; ++e) num[e] = 0.f;
#pragma unroll
    for (int z = 0; z < MAXS; ++z) {
      const float wz = __shfl(w, z, 64);  // 0 for splits past S
#pragma unroll
      for (int e = 0; e < DV; ++e) num[e] = fmaf(v[e][z], wz, num[e]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int e = 0; e < DV; ++e)
      if (lane + 64 * e < D) out[out_at(lane + 64 * e)] = Elem<T>::from_f32(rejected ? 0.f : num[e] * inv);
  };
  if constexpr (MAXS <= 2) {
    // few splits: every head's loads go out before any store (head by head,
    // a head's loads would queue behind the previous head's stores, which
    // may alias them as far as the compiler knows); heads past n_q re-read
    // the last head and are not stored.  (With more splits the wider loads
    // of all heads at once measured slower.)
    float m_l[HPW], l_l[HPW], v[HPW][DV][MAXS];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) load_head(min(h0 + hh, a.n_q - 1), m_l[hh], l_l[hh], v[hh]);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (h0 + hh >= a.n_q) break;
      merge_store(h0 + hh, m_l[hh], l_l[hh], v[hh]);
    }
  } else {
    // HPW heads per wave, unrolled so that their loads are in flight together
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      if (h >= a.n_q) break;
      float m_l, l_l, v[DV][MAXS];
      load_head(h, m_l, l_l, v);
      merge_store(h, m_l, l_l, v);
    }
  }
}

template <int D>
void launch_mfma(const AttnArgs& a, dim3 grid, hipStream_t s) {
  // The LDS-DMA ring whenever a split's page numbers fit in LDS, else the
  // register-staged kernel reading the block table (64-dim heads: two
  // workgroups per CU; 128-dim heads: one, with a deeper register prefetch,
  // as two would spill).  The ring keeps three stages for 64-dim heads; for
  // 128-dim heads two stages (68 KiB of LDS, at most 128 VGPRs) let two
  // workgroups share a CU where three stages fit only one (Qwen-shaped c=16,
  // K=7: 79.8 -> 77.8 us).
  constexpr int DEPTH = D == 64 ? 2 : 3, OCC = D == 64 ? 4 : 2;
  if (a.max_blocks <= (kAttnMaxPages - 8) * a.splits)
    hipLaunchKernelGGL((attn_ring_kernel<D, D == 128 ? 2 : 3>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, DEPTH, OCC, false>), grid, dim3(512), 0, s, a);
}

// Split merge: four waves per workgroup, HPW heads per wave, split loads
// bounded by the next power of two at or above the split count.
template <typename T, int D, int MAXS>
void launch_combine_s(const AttnArgs& a, hipStream_t s) {
  constexpr int HPW = 2;
  const dim3 grid(a.N, (a.n_q + 4 * HPW - 1) / (4 * HPW));
  hipLaunchKernelGGL((attn_combine_kernel<T, D, MAXS, HPW>), grid, dim3(256), 0, s, a);
}
template <typename T, int D>
void launch_combine(const AttnArgs& a, hipStream_t s) {
  if (a.splits <= 1) launch_combine_s<T, D, 1>(a, s);
  else if (a.splits <= 2) launch_combine_s<T, D, 2>(a, s);
  else if (a.splits <= 4) launch_combine_s<T, D, 4>(a, s);
  else if (a.splits <= 8) launch_combine_s<T, D, 8>(a, s);
  else launch_combine_s<T, D, kAttnMaxSplits>(a, s);
}

template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  if (a.splits < 1 || a.splits > kAttnMaxSplits || a.d > 128) return hipErrorInvalidValue;
  dim3 grid(a.splits, a.n_kv, a.c);
  if (sizeof(T) == 2 && (a.d == 64 || a.d == 128)) {
    if (a.d == 64)
      launch_mfma<64>(a, grid, s);
    else
      launch_mfma<128>(a, grid, s);
  } else {
    switch (a.d) {
      case 16: hipLaunchKernelGGL((attn_split_kernel<T, 16>), grid, dim3(256), 0, s, a); break;
      case 32: hipLaunchKernelGGL((attn_split_kernel<T, 32>), grid, dim3(256), 0, s, a); break;
      case 64: hipLaunchKernelGGL((attn_split_kernel<T, 64>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((attn_split_kernel<T, 128>), grid, dim3(256), 0, s, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.d) {
    case 16: launch_combine<T, 16>(a, s); break;
    case 32: launch_combine<T, 32>(a, s); break;
    case 64: launch_combine<T, 64>(a, s); break;
    default: launch_combine<T, 128>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.out_group < 0 || (a.out_group > 0 && (a.n_q * a.d) % 32 != 0)) return hipErrorInvalidValue;
  return a.dtype == DType::F32 ? launch_t<float>(a, s) : launch_t<bf16_t>(a, s);
}

}  // namespace pe
