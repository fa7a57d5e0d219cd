// RMSNorm in front of the fused LoRA MLP: forward, re-application from the
// saved statistics, and backward.
//
// The norm is one of the hand-written forward+backward kernels of the
// training path in "Unsloth 深度分析报告" (section 关键设计决策), and
// "Unsloth支持哪些模型？主流LLM兼容性一览" (section 4.2) has its backward
// reuse the statistics of the forward instead of recomputing them. With
// rstd_t = (mean_h x_th^2 + eps)^(-1/2) and a frozen weight gamma:
//   forward   xn = x * rstd * gamma (rstd saved, one fp32 per token row)
//   apply     xn from the saved rstd (no reduction): the backward's copy of
//             the MLP's input, bitwise equal to the forward's
//   backward  dx = rstd * (gamma g - xhat * mean_h(gamma g xhat)), xhat = x rstd
//
// All three are HBM-bound row streams (2-3 bytes moved per FLOP), so the
// layout is for bandwidth: one wave per token row, four rows per workgroup,
// lane l holding the 16-byte chunks l, l + 64, l + 128, ... of its row (each
// chunk index is one contiguous 1 KB access of the wave). Up to NC chunks per
// lane stay in registers between the reduction and the output pass; wider
// rows (NC == 0) read the row a second time. Row sums are formed in a fixed
// order (per lane in chunk order, then a butterfly across the wave), so every
// result is deterministic.
#include "common.h"
#include "kernels.h"

namespace lmlp {

namespace {

template <typename T> struct rowchunk;
template <> struct rowchunk<bf16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& c, float* v) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static uint4 pack(const float* v) {
    return make_uint4(pack_bf16x2_pk(v[0], v[1]), pack_bf16x2_pk(v[2], v[3]), pack_bf16x2_pk(v[4], v[5]),
                      pack_bf16x2_pk(v[6], v[7]));
  }
};
template <> struct rowchunk<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& c, float* v) {
    v[0] = __uint_as_float(c.x);
    v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z);
    v[3] = __uint_as_float(c.w);
  }
  __device__ static uint4 pack(const float* v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ uint4 ld16(const void* base, int64_t chunk) {
  return reinterpret_cast<const uint4*>(base)[chunk];
}
__device__ __forceinline__ void st16(void* base, int64_t chunk, const uint4& v) {
  reinterpret_cast<uint4*>(base)[chunk] = v;
}

// xn = x * rs * gamma for one chunk
template <typename T>
__device__ __forceinline__ uint4 scale_chunk(const uint4& xc, const uint4& gc, float rs) {
  constexpr int N = rowchunk<T>::N;
  float xv[N], gv[N];
  rowchunk<T>::unpack(xc, xv);
  rowchunk<T>::unpack(gc, gv);
#pragma unroll
  for (int i = 0; i < N; ++i) xv[i] = xv[i] * rs * gv[i];
  return rowchunk<T>::pack(xv);
}

// forward (mode NORM_FWD) or re-application (NORM_APPLY)
template <typename T, int NC>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(NormParams p) {
  constexpr int N = rowchunk<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.T) return;
  const int64_t nch = p.H / N;  // 16-byte chunks per row
  const char* xr = static_cast<const char*>(p.x) + row * p.H * static_cast<int64_t>(sizeof(T));
  char* yr = static_cast<char*>(p.xn) + row * p.H * static_cast<int64_t>(sizeof(T));
  // the row and the matching gamma chunks are loaded together, before the
  // reduction, so each wave waits for memory once
  uint4 xc[NC > 0 ? NC : 1], wc[NC > 0 ? NC : 1];
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t k = c * 64 + lane;
      xc[c] = k < nch ? ld16(xr, k) : zero4();
      wc[c] = k < nch ? ld16(p.gamma, k) : zero4();
    }
  }
  float rs;
  if (p.mode == NORM_APPLY) {
    rs = p.rstd[row];
  } else {
    float ss = 0.f;
    if constexpr (NC > 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float v[N];
        rowchunk<T>::unpack(xc[c], v);
#pragma unroll
        for (int i = 0; i < N; ++i) ss += v[i] * v[i];
      }
    } else {
      for (int64_t k = lane; k < nch; k += 64) {
        float v[N];
        rowchunk<T>::unpack(ld16(xr, k), v);
#pragma unroll
        for (int i = 0; i < N; ++i) ss += v[i] * v[i];
      }
    }
    ss = wave_sum(ss);
    rs = rsqrtf(ss / static_cast<float>(p.H) + p.eps);
    if (lane == 0) p.rstd[row] = rs;
  }
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t k = c * 64 + lane;
      if (k < nch) st16(yr, k, scale_chunk<T>(xc[c], wc[c], rs));
    }
  } else {
    for (int64_t k = lane; k < nch; k += 64) st16(yr, k, scale_chunk<T>(ld16(xr, k), ld16(p.gamma, k), rs));
  }
}

// backward: dx = rs * (gamma g - xhat * c), c = mean(gamma g xhat); g may alias dx
template <typename T, int NC>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(NormParams p) {
  constexpr int N = rowchunk<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.T) return;
  const int64_t nch = p.H / N;
  const int64_t off = row * p.H * static_cast<int64_t>(sizeof(T));
  const char* xr = static_cast<const char*>(p.x) + off;
  const char* gr = static_cast<const char*>(p.g) + off;
  char* dr = static_cast<char*>(p.dx) + off;
  const float rs = p.rstd[row];
  // one chunk's contribution to the dot
  auto dot_chunk = [&](const uint4& xc, const uint4& gc, const uint4& wc) {
    float xv[N], gv[N], wv[N], d = 0.f;
    rowchunk<T>::unpack(xc, xv);
    rowchunk<T>::unpack(gc, gv);
    rowchunk<T>::unpack(wc, wv);
#pragma unroll
    for (int i = 0; i < N; ++i) d += (gv[i] * wv[i]) * (xv[i] * rs);
    return d;
  };
  auto out_chunk = [&](const uint4& xc, const uint4& gc, const uint4& wc, float cm) {
    float xv[N], gv[N], wv[N];
    rowchunk<T>::unpack(xc, xv);
    rowchunk<T>::unpack(gc, gv);
    rowchunk<T>::unpack(wc, wv);
#pragma unroll
    for (int i = 0; i < N; ++i) xv[i] = rs * ((gv[i] * wv[i]) - (xv[i] * rs) * cm);
    return rowchunk<T>::pack(xv);
  };
  float dot = 0.f;
  if constexpr (NC > 0) {
    uint4 xc[NC], gc[NC], wc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t k = c * 64 + lane;
      xc[c] = k < nch ? ld16(xr, k) : zero4();
      gc[c] = k < nch ? ld16(gr, k) : zero4();
      wc[c] = k < nch ? ld16(p.gamma, k) : zero4();
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) dot += dot_chunk(xc[c], gc[c], wc[c]);  // zero past the row
    const float cm = wave_sum(dot) / static_cast<float>(p.H);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t k = c * 64 + lane;
      if (k < nch) st16(dr, k, out_chunk(xc[c], gc[c], wc[c], cm));
    }
  } else {
    for (int64_t k = lane; k < nch; k += 64) dot += dot_chunk(ld16(xr, k), ld16(gr, k), ld16(p.gamma, k));
    const float cm = wave_sum(dot) / static_cast<float>(p.H);
    for (int64_t k = lane; k < nch; k += 64) st16(dr, k, out_chunk(ld16(xr, k), ld16(gr, k), ld16(p.gamma, k), cm));
  }
}

template <typename T>
hipError_t launch_typed(const NormParams& p, hipStream_t st) {
  const int64_t nch = p.H / rowchunk<T>::N;
  const int64_t per_lane = (nch + 63) / 64;
  const dim3 grid(static_cast<unsigned>((p.T + 3) / 4)), block(256);
  const bool bwd = p.mode == NORM_BWD;
#define LMLP_NORM_LAUNCH(NCV)                                                             \
  if (bwd) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, NCV>), grid, block, 0, st, p);      \
  else hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, NCV>), grid, block, 0, st, p);
  if (per_lane <= 1) { LMLP_NORM_LAUNCH(1) }
  else if (per_lane <= 2) { LMLP_NORM_LAUNCH(2) }
  else if (per_lane <= 4) { LMLP_NORM_LAUNCH(4) }
  else if (per_lane <= 8) { LMLP_NORM_LAUNCH(8) }
  else if (per_lane <= 16) { LMLP_NORM_LAUNCH(16) }
  else { LMLP_NORM_LAUNCH(0) }
#undef LMLP_NORM_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const NormParams& p, int dtype_bf16, hipStream_t stream) {
  if (p.T <= 0 || p.H <= 0) return hipSuccess;
  return dtype_bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace lmlp
