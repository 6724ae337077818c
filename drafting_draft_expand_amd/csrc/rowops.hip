// Row-wise kernels of the drafter pass: fc input assembly, RMSNorm, RoPE with
// the paged KV write, LM-head argmax merge and greedy acceptance.
#include "common.h"

namespace pe {
namespace {

// u[r] = [embed[ids[r]] ; draft_hidden[r]]  -- the concatenation of the
// "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding in vLLM"
// Input_i equation (token embedding first, hidden state second).
__global__ __launch_bounds__(256) void fc_input_kernel(int H_bytes, const int32_t* ids, const char* embed,
                                                       const char* hidden, char* out) {
  const int r = blockIdx.x;
  const int hv = H_bytes / 16;
  const char* e = embed + static_cast<int64_t>(ids[r]) * H_bytes;
  const char* h = hidden + static_cast<int64_t>(r) * H_bytes;
  char* o = out + static_cast<int64_t>(r) * 2 * H_bytes;
  for (int v = threadIdx.x; v < 2 * hv; v += blockDim.x) {
    const char* src = v < hv ? e + v * 16 : h + (v - hv) * 16;
    store16(o + v * 16, load16(src));
  }
}

// four consecutive elements as fp32 (p 8-byte aligned for bf16, 16 for fp32)
template <typename T>
__device__ __forceinline__ f32x4 load4_f32(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    return f32x4{bf16_to_f32(static_cast<bf16_t>(r.x & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(r.x >> 16)),
                 bf16_to_f32(static_cast<bf16_t>(r.y & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(r.y >> 16))};
  }
}

// out[i] = x[row] / sqrt(mean(x[row]^2) + eps) * gain, rounded to the operand
// dtype; one workgroup per row, row = row_idx ? row_idx[i] : i.  With NS > 0
// the row is first completed from the split partials of the projection that
// produced it, x[row] = (accumulate ? x[row] : 0) + part[0][row] + part[1][row]
// + ..., summed in split order and written back as the new residual row.
// Every thread holds at most two 16-byte pieces of the row and issues all of
// their loads (residual and partials) before the first add.
template <typename T, int NS>
__global__ __launch_bounds__(1024) void rmsnorm_kernel(int H, const int32_t* __restrict__ row_idx,
                                                       float* __restrict__ x, const T* __restrict__ gain,
                                                       float eps, T* __restrict__ out,
                                                       const int32_t* __restrict__ live,
                                                       const float* __restrict__ part, int64_t part_stride,
                                                       int accumulate, int out_group, RopeTable rt) {
  __shared__ float wave_ss[16];
  const int i = blockIdx.x;
  if (rt.out && static_cast<int>(threadIdx.x) < rt.half) {
    float c, s;
    rope_cos_sin(rt.pos[i], rt.freq.inv[threadIdx.x], c, s);
    rt.out[static_cast<int64_t>(i) * rt.half + threadIdx.x] = make_float2(c, s);
  }
  const int r = row_idx ? row_idx[i] : i;
  f32x4* xr = reinterpret_cast<f32x4*>(x + static_cast<int64_t>(r) * H);
  const int nv = H / 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 keep[2];
  float ss = 0.f;
  int nlive;
  // the gains are requested with the row, so that their latency overlaps the
  // row's and the reduction
  f32x4 gv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    gv[u] = load4_f32(gain + 4 * min(static_cast<int>(threadIdx.x + blockDim.x * u), nv - 1));
  {
    f32x4 xv[2], pv[2][NS > 0 ? NS : 1];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int v = min(static_cast<int>(threadIdx.x + blockDim.x * u), nv - 1);
      xv[u] = NS == 0 || accumulate ? xr[v] : zero;
#pragma unroll
      for (int z = 0; z < NS; ++z)
        pv[u][z] = reinterpret_cast<const f32x4*>(part + z * part_stride + static_cast<int64_t>(r) * H)[v];
    }
    // padding row of the compacted layout (nothing stored): the live count is
    // requested only now, after the row's loads (the compiler barrier keeps it
    // there), and tested once the row has arrived, so the row does not wait
    // for it (a scalar load waited for early would hold back every later one)
    asm volatile("" : : : "memory");
    nlive = live ? *live : 0x7fffffff;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 q = xv[u];
#pragma unroll
      for (int z = 0; z < NS; ++z) q += pv[u][z];
      const bool mine = static_cast<int>(threadIdx.x + blockDim.x * u) < nv;
      q = mine ? q : zero;
      keep[u] = q;
      ss += q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3];
    }
  }
  // (the sum above is formed on every path, so the row loads stay ahead of the test)
  asm volatile("" : : "v"(ss));
  if (i >= nlive) {
    // (the gains, still in flight, are waited for before the wave ends)
    asm volatile("" : : "v"(gv[0]), "v"(gv[1]));
    return;
  }
  if (NS > 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (static_cast<int>(threadIdx.x + blockDim.x * u) < nv) xr[threadIdx.x + blockDim.x * u] = keep[u];
  }
  ss = wave_sum(ss);
  const int nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) wave_ss[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = 0.f;
  for (int w = 0; w < nw; ++w) ss += wave_ss[w];
  const float scale = 1.f / sqrtf(ss / static_cast<float>(H) + eps);
  // row-major, or tile-major in groups of out_group rows: element k of row i at
  // ((i / G) * (H / 32) + k / 32) * G * 32 + (i % G) * 32 + k % 32 (a piece of
  // four never straddles a 32-wide slice)
  const int64_t row_base = out_group > 0 ? static_cast<int64_t>(i / out_group) * out_group * H + (i % out_group) * 32
                                         : static_cast<int64_t>(i) * H;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int v = threadIdx.x + blockDim.x * u;
    if (v >= nv) continue;
    const f32x4 q = keep[u];
    const int k = 4 * v;
    T* o = out + row_base + (out_group > 0 ? static_cast<int64_t>(k / 32) * out_group * 32 + k % 32 : k);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = Elem<T>::from_f32(q[e] * scale * gv[u][e]);
  }
}

// Rotate-half RoPE of q and k at the row's position, q stored as the attention
// operand, k and v written to the paged cache at the row's slot.  Rows with
// slot -1 (rejected, "P-EAGLE: Parallel Speculative Decoding in vLLM", KV Cache
// and CUDA Graphs) write nothing.
template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(RopeArgs a) {
  const int r = blockIdx.x;
  const int half = a.d / 2;
  const int heads = a.n_q + 2 * a.n_kv;
  const int p = blockIdx.y * blockDim.x + threadIdx.x;
  if (p >= heads * half) return;
  if (a.rejected[r]) return;
  const int head = p / half;
  const int j = p - head * half;
  const float* src = a.qkv + static_cast<int64_t>(r) * heads * a.d + head * a.d;
  float x1 = src[j], x2 = src[j + half];
  if (head < a.n_q + a.n_kv) {
    float c, s;
    rope_cos_sin(a.pos[r], a.freq.inv[j], c, s);
    const float y1 = x1 * c - x2 * s;
    const float y2 = x2 * c + x1 * s;
    x1 = y1;
    x2 = y2;
  }
  if (head < a.n_q) {
    T* q = static_cast<T*>(a.q_out) + static_cast<int64_t>(r) * a.n_q * a.d + head * a.d;
    q[j] = Elem<T>::from_f32(x1);
    q[j + half] = Elem<T>::from_f32(x2);
    return;
  }
  const int64_t slot = a.slot[r];
  if (slot < 0) return;
  const bool is_k = head < a.n_q + a.n_kv;
  const int g = is_k ? head - a.n_q : head - a.n_q - a.n_kv;
  const int64_t blk = slot / a.block_size;
  const int off = static_cast<int>(slot - blk * a.block_size);
  T* dst = static_cast<T*>(is_k ? a.k_cache : a.v_cache) +
           ((blk * a.n_kv + g) * a.block_size + off) * a.d;
  dst[j] = Elem<T>::from_f32(x1);
  dst[j + half] = Elem<T>::from_f32(x2);
}

// Merge the per-workgroup LM-head candidates of each sampled row: token =
// best id (lowest id on ties), gap = best minus runner-up logit.  The merge is
// order-independent; 256 threads read up to 1024 candidates per round, all
// loads of a round issued before the first merge.
__global__ __launch_bounds__(256) void argmax_finalize_kernel(int parts, const Top2* partials, int32_t* tokens,
                                                              float* gap) {
  __shared__ Top2 red[4];
  const int s = blockIdx.x;
  const Top2* row = partials + static_cast<int64_t>(s) * parts;
  Top2 best = top2_empty();
  for (int p0 = 0; p0 < parts; p0 += 1024) {
    Top2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = row[min(p0 + static_cast<int>(threadIdx.x) + 256 * u, parts - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (p0 + static_cast<int>(threadIdx.x) + 256 * u < parts) best = top2_merge(best, v[u]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Top2 o;
    o.v1 = __shfl_xor(best.v1, off, 64);
    o.i1 = __shfl_xor(best.i1, off, 64);
    o.v2 = __shfl_xor(best.v2, off, 64);
    o.pad = 0;
    best = top2_merge(best, o);
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    best = top2_merge(top2_merge(red[0], red[1]), top2_merge(red[2], red[3]));
    tokens[s] = best.i1;
    if (gap) gap[s] = best.v1 - best.v2;
  }
}

// Greedy acceptance: longest prefix where draft == target, then the bonus
// token ("P-EAGLE: Parallel Speculative Decoding in vLLM", Acceptance Length).
// The K comparisons have no early exit, so all loads go out together.
__global__ __launch_bounds__(256) void accept_kernel(int c, int K, const int32_t* draft, const int32_t* target,
                                                     int32_t* acc, int32_t* bonus) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= c) return;
  const int32_t* d = draft + static_cast<int64_t>(i) * K;
  const int32_t* t = target + static_cast<int64_t>(i) * (K + 1);
  int n = K;
  int32_t b = t[K];
#pragma unroll 8
  for (int k = 0; k < K; ++k) {
    const int32_t tk = t[k];
    const bool miss = d[k] != tk;
    if (n == K && miss) {
      n = k;
      b = tk;
    }
  }
  acc[i] = n;
  bonus[i] = b;
}

}  // namespace

hipError_t launch_build_fc_input(DType dt, int N, int H, const int32_t* ids, const void* embed,
                                 const void* draft_hidden, void* out, hipStream_t s) {
  hipLaunchKernelGGL(fc_input_kernel, dim3(N), dim3(256), 0, s, H * elem_bytes(dt), ids,
                     static_cast<const char*>(embed), static_cast<const char*>(draft_hidden),
                     static_cast<char*>(out));
  return hipGetLastError();
}

namespace {
// Compute units of the current device (queried once per device).
constexpr int kMaxWavesPerCu = 32;
int device_cus() {
  static int cached[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 256;
  if (cached[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cached[dev] = c;
  }
  return cached[dev];
}

template <typename T, int NS>
void launch_rmsnorm_t(int rows, int H, const int32_t* row_idx, float* x, const void* gain, float eps, void* out,
                      hipStream_t s, const int32_t* live, const float* part, int64_t stride, bool accumulate,
                      int out_group, const RopeTable& rt) {
  const int nv = H / 4;
  int threads = ((nv + 1) / 2 + 63) / 64 * 64;  // at most two pieces per thread
  if (threads < 64) threads = 64;
  if (nv <= 1024) {
    // one piece per thread while that fits, unless two per thread (half the
    // waves per row) keep every row resident in fewer rounds: 896 rows of
    // 2880 take two rounds at 12 waves per row and one at 6
    const int one = (nv + 63) / 64 * 64;
    auto rounds = [&](int th) {
      const int per_cu = kMaxWavesPerCu / (th / 64);
      const int64_t slots = static_cast<int64_t>(device_cus()) * (per_cu > 0 ? per_cu : 1);
      return (rows + slots - 1) / slots;
    };
    threads = rounds(threads) < rounds(one) ? threads : one;
  }
  if (threads < rt.half) threads = (rt.half + 63) / 64 * 64;
  hipLaunchKernelGGL((rmsnorm_kernel<T, NS>), dim3(rows), dim3(threads), 0, s, H, row_idx, x,
                     static_cast<const T*>(gain), eps, static_cast<T*>(out), live, part, stride, int(accumulate),
                     out_group, rt);
}

template <typename T>
hipError_t launch_rmsnorm_dt(int rows, int H, const int32_t* row_idx, float* x, const void* gain, float eps,
                             void* out, hipStream_t s, const int32_t* live, const float* part, int nsplit,
                             int64_t stride, bool accumulate, int out_group, const RopeTable& rt) {
  const int og = out_group;
  switch (nsplit) {
    case 0: launch_rmsnorm_t<T, 0>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 1: launch_rmsnorm_t<T, 1>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 2: launch_rmsnorm_t<T, 2>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 3: launch_rmsnorm_t<T, 3>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 4: launch_rmsnorm_t<T, 4>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 5: launch_rmsnorm_t<T, 5>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 6: launch_rmsnorm_t<T, 6>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 7: launch_rmsnorm_t<T, 7>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    case 8: launch_rmsnorm_t<T, 8>(rows, H, row_idx, x, gain, eps, out, s, live, part, stride, accumulate, og, rt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_rmsnorm(DType dt, int rows, int H, const int32_t* row_idx, float* x, const void* gain,
                          float eps, void* out, hipStream_t s, const int32_t* live, const float* part, int nsplit,
                          int part_rows, bool accumulate, int out_group, const RopeTable* rope) {
  if (H % 4 != 0 || H > kMaxHidden || rows <= 0) return hipErrorInvalidValue;
  if (nsplit > 0 && !part) return hipErrorInvalidValue;
  if (out_group < 0 || (out_group > 0 && H % 32 != 0)) return hipErrorInvalidValue;
  RopeTable rt{};
  if (rope && rope->out) {
    if (rope->half < 1 || rope->half > 64 || !rope->pos) return hipErrorInvalidValue;
    rt = *rope;
  }
  const int64_t stride = static_cast<int64_t>(part_rows) * H;
  if (dt == DType::F32)
    return launch_rmsnorm_dt<float>(rows, H, row_idx, x, gain, eps, out, s, live, part, nsplit, stride, accumulate,
                                    out_group, rt);
  return launch_rmsnorm_dt<bf16_t>(rows, H, row_idx, x, gain, eps, out, s, live, part, nsplit, stride, accumulate,
                                   out_group, rt);
}

hipError_t launch_rope_kvwrite(const RopeArgs& a, hipStream_t s) {
  const int pairs = (a.n_q + 2 * a.n_kv) * (a.d / 2);
  dim3 grid(a.N, (pairs + 255) / 256);
  if (a.dtype == DType::F32)
    hipLaunchKernelGGL(rope_kv_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rope_kv_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(int S, int parts, const Top2* partials, int32_t* tokens, float* gap,
                                  hipStream_t s) {
  if (parts < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(S), dim3(256), 0, s, parts, partials, tokens, gap);
  return hipGetLastError();
}

hipError_t launch_accept(int c, int K, const int32_t* draft, const int32_t* target, int32_t* acc,
                         int32_t* bonus, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3((c + 255) / 256), dim3(256), 0, s, c, K, draft, target, acc, bonus);
  return hipGetLastError();
}

}  // namespace pe
