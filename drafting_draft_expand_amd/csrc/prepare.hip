// Batch expansion + hidden-state placement for one parallel-draft round.
//
// "P-EAGLE: Parallel Speculative Decoding in vLLM", vLLM Implementation
// Details / Fused Triton Kernel: the draft batch differs in shape from the
// verify batch because of the MASK placeholders, so ids, positions, the bonus
// token, the MASK fill and the rejected/masked/hidden-map metadata are rebuilt
// on the GPU in a single launch.  Same page, Hidden State Management, and the
// listing in "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding
// in vLLM", vLLM implementation details: target hidden rows move to their new
// rows and the learned shared hidden state fills the MASK rows.  KV Cache and
// CUDA Graphs: rejected rows get slot -1.  The compacted layout drops the
// rejected rows instead (a + K rows per sequence) and parks inert padding rows
// after the live ones, so buffer shapes stay those of the fixed layout.
//
// One launch, grid (sequence, column chunk + 1), 256 threads:
//   * every block derives its sequence's first verified row (and, compacted,
//     its first draft row and the live total) in one block-wide reduction over
//     the preceding query lengths, with its own L and a loaded alongside;
//   * the last block of each sequence writes the per-row metadata, so that
//     no hidden-row copy waits behind the metadata's loads and stores;
//   * every other block copies its column slice of all L+K-1 hidden rows of
//     the sequence with 16-byte loads/stores, reading either the target row the
//     draft row maps from or h_shared.  Each output row is written once, so
//     placement and broadcast form a single gather with no ordering hazard.
#include "common.h"

namespace pe {
namespace {

// Block-wide sums over j < n of v[j], and (when w is set) of w[j] for j < n
// and j < nw; every thread gets all three.
struct PrefixSums {
  int v, w_lo, w_all;
};
__device__ __forceinline__ PrefixSums block_prefix_sums(const int32_t* v, int n, const int32_t* w, int nw) {
  __shared__ int part[4][3];
  int s = 0, lo = 0, all = 0;
  for (int j = threadIdx.x; j < n; j += blockDim.x) s += v[j];
  if (w) {
    for (int j = threadIdx.x; j < nw; j += blockDim.x) {
      const int x = w[j];
      all += x;
      lo += j < n ? x : 0;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s += __shfl_xor(s, off, 64);
    lo += __shfl_xor(lo, off, 64);
    all += __shfl_xor(all, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    part[threadIdx.x >> 6][0] = s;
    part[threadIdx.x >> 6][1] = lo;
    part[threadIdx.x >> 6][2] = all;
  }
  __syncthreads();
  PrefixSums r;
  r.v = part[0][0] + part[1][0] + part[2][0] + part[3][0];
  r.w_lo = part[0][1] + part[1][1] + part[2][1] + part[3][1];
  r.w_all = part[0][2] + part[1][2] + part[2][2] + part[3][2];
  return r;
}

__global__ __launch_bounds__(256) void prepare_kernel(PrepareArgs a, int row_bytes, int vecs_per_row,
                                                      int vecs_per_chunk) {
  const int i = blockIdx.x;
  const int K = a.K;
  // this sequence's own values first: their loads overlap the reduction's
  const int L = a.query_lens[i];
  const int acc = a.num_accepted[i];
  const PrefixSums ps = block_prefix_sums(a.query_lens, i, a.compact ? a.num_accepted : nullptr, a.c);
  const int s = ps.v;
  // fixed layout: L + K - 1 rows per sequence (rejected rows kept, inert);
  // compacted: a + K rows (rejected rows dropped), then inert padding rows up
  // to the fixed total, sequence i padding as many rows as it dropped
  const int D_fixed = s + i * (K - 1);
  int D = D_fixed, rows = L + K - 1, live = a.N, pad0 = 0, npad = 0;
  if (a.compact) {
    D = ps.w_lo + i * K;
    rows = acc + K;
    live = ps.w_all + a.c * K;
    pad0 = live + (D_fixed - D);
    npad = L - 1 - acc;
  }

  if (blockIdx.y == gridDim.y - 1) {
    const int bonus = a.bonus_ids[i];
    const int base = a.target_pos[s + acc];
    const int bs = a.block_size;
    const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
    for (int r = threadIdx.x; r < rows; r += blockDim.x) {
      int id, pos;
      uint8_t masked = 0, rejected = 0;
      if (r <= acc) {                       // accepted rows, then the bonus row
        id = r < acc ? a.target_ids[s + r + 1] : bonus;
        pos = a.target_pos[s + r];
      } else if (r < acc + K) {             // K-1 parallel-drafting MASK rows
        id = a.mask_id;
        pos = base + (r - acc);
        masked = 1;
      } else {                              // rejected verified rows
        const int j = r - (K - 1);
        id = j + 1 < L ? a.target_ids[s + j + 1] : bonus;
        pos = a.target_pos[s + j];
        rejected = 1;
      }
      const int row = D + r;
      a.draft_ids[row] = id;
      a.draft_pos[row] = pos;
      a.is_masked[row] = masked;
      a.is_rejected[row] = rejected;
      a.slot_mapping[row] =
          rejected ? int64_t(-1) : int64_t(bt[pos / bs]) * bs + pos % bs;
    }
    for (int r = threadIdx.x; r < npad; r += blockDim.x) {
      const int row = pad0 + r;             // padding: never written, attended or sampled
      a.draft_ids[row] = bonus;
      a.draft_pos[row] = 0;
      a.is_masked[row] = 0;
      a.is_rejected[row] = 1;
      a.slot_mapping[row] = int64_t(-1);
    }
    for (int j = threadIdx.x; j < L; j += blockDim.x)
      a.hidden_map[s + j] = j <= acc ? D + j : (a.compact ? -1 : D + j + K - 1);
    for (int k = threadIdx.x; k < K; k += blockDim.x) a.sample_idx[i * K + k] = D + acc + k;
    if (threadIdx.x == 0) {
      a.cu_draft[i] = D;
      a.kv_lens[i] = base + K;
      if (i == a.c - 1) a.cu_draft[a.c] = live;
    }
    return;
  }

  // hidden placement: gather of 16-byte vectors for this block's column slice
  const int v0 = blockIdx.y * vecs_per_chunk;
  const int width = min(vecs_per_chunk, vecs_per_row - v0);
  if (width <= 0) return;
  const char* th = static_cast<const char*>(a.target_hidden);
  const char* hs = static_cast<const char*>(a.h_shared);
  char* out = static_cast<char*>(a.draft_hidden);
  // four 16-byte pieces per thread and round, all loads issued before the
  // stores (pieces past the end re-read the last one and are not stored)
  const int total = rows * width;
  constexpr int UP = 4;
  for (int f0 = threadIdx.x; f0 < total; f0 += blockDim.x * UP) {
    u32x4 val[UP];
    int64_t dst[UP];
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int f = min(f0 + u * static_cast<int>(blockDim.x), total - 1);
      const int r = f / width;
      const int v = v0 + f - r * width;
      const char* src;
      if (r > acc && r < acc + K) {
        src = hs + v * 16;
      } else {
        const int j = r <= acc ? r : r - (K - 1);
        src = th + static_cast<int64_t>(s + j) * row_bytes + v * 16;
      }
      val[u] = load16(src);
      dst[u] = static_cast<int64_t>(D + r) * row_bytes + v * 16;
    }
#pragma unroll
    for (int u = 0; u < UP; ++u)
      if (f0 + u * static_cast<int>(blockDim.x) < total) store16(out + dst[u], val[u]);
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int f = threadIdx.x; f < npad * width; f += blockDim.x) {
    const int r = f / width;
    store16(out + static_cast<int64_t>(pad0 + r) * row_bytes + (v0 + f - r * width) * 16, zero);
  }
}

// Device-side preconditions of the expansion, one block per sequence.  Every
// value is range-checked before it is used as an index, so malformed input
// only sets bits.
__global__ __launch_bounds__(256) void check_batch_kernel(CheckArgs a) {
  __shared__ int flags;
  __shared__ int part[4];
  const int i = blockIdx.x;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  // first verified row of sequence i (lengths clamped into [0, T] for the sum)
  int s = 0;
  for (int j = threadIdx.x; j < i; j += blockDim.x) s += min(max(a.query_lens[j], 0), a.T);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  s = part[0] + part[1] + part[2] + part[3];
  int bits = 0;
  if (i == 0 && threadIdx.x == 0) {
    int64_t total = 0;
    for (int j = 0; j < a.c; ++j) total += a.query_lens[j];
    if (total != a.T) bits |= kCheckQueryLen;
  }
  const int L = a.query_lens[i];
  const int acc = a.num_accepted[i];
  const int bonus = a.bonus_ids[i];
  bool ok = L >= 1 && s + L <= a.T;
  if (!ok) bits |= kCheckQueryLen;
  if (ok && (acc < 0 || acc > L - 1)) {
    bits |= kCheckAccepted;
    ok = false;
  }
  if (threadIdx.x == 0 && (bonus < 0 || bonus >= a.V)) bits |= kCheckTokenId;
  if (ok) {
    const int p0 = a.target_pos[s];
    for (int j = threadIdx.x; j < L; j += blockDim.x) {
      const int id = a.target_ids[s + j];
      if (id < 0 || id >= a.V) bits |= kCheckTokenId;
      const int p = a.target_pos[s + j];
      if (p < 0 || p != p0 + j) bits |= kCheckPosition;
    }
    // every page the pass reads or writes: positions 0 .. target_pos[first + a_i] + K - 1
    const int64_t last = static_cast<int64_t>(a.target_pos[s + acc]) + a.K - 1;
    if (last < 0 || last / 16 >= a.max_blocks) {
      bits |= kCheckBlockTable;
    } else {
      const int32_t* bt = a.block_table + static_cast<int64_t>(i) * a.max_blocks;
      for (int q = threadIdx.x; q <= static_cast<int>(last / 16); q += blockDim.x)
        if (bt[q] < 0) bits |= kCheckBlockTable;
    }
  }
  if (bits) atomicOr(&flags, bits);
  __syncthreads();
  if (threadIdx.x == 0 && flags) atomicOr(a.error_bits, flags);
}

}  // namespace

hipError_t launch_check_batch(const CheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(check_batch_kernel, dim3(a.c), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prepare(const PrepareArgs& a, hipStream_t stream) {
  const int row_bytes = a.H * elem_bytes(a.dtype);
  const int vecs = row_bytes / 16;
  // enough blocks to cover the chip even at concurrency 1
  int chunks = (512 + a.c - 1) / a.c;
  chunks = chunks < 1 ? 1 : chunks;
  const int max_chunks = (vecs + 7) / 8;
  if (chunks > max_chunks) chunks = max_chunks;
  const int per_chunk = (vecs + chunks - 1) / chunks;
  chunks = (vecs + per_chunk - 1) / per_chunk;
  // the column chunks, then one metadata block per sequence
  dim3 grid(a.c, chunks + 1);
  hipLaunchKernelGGL(prepare_kernel, grid, dim3(256), 0, stream, a, row_bytes, vecs, per_chunk);
  return hipGetLastError();
}

}  // namespace pe
