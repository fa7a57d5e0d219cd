// Rank-r side products of the fused LoRA MLP and small helpers.
//
// The adapter terms of "Unsloth 深度分析报告" (section 创新之处: the gate, up
// and down LoRA paths fused into one forward/backward) need, besides the big
// GEMMs, thin products with the rank-r factors:
//   row projections (contract the long feature axis of every token row):
//     X A_gu^T, Z A_d^T, dY B_d, dG B_g, dU B_u            -> [T, r]
//   column projections (contract the token axis):
//     dY^T Pd, dG^T P_g, dU^T P_u, Z^T Q_d, X^T Q_gu        -> [H or I, r]
// Both are HBM-bound streams over one [T, K] activation; they run on MFMA
// because at r >= 16 their arithmetic intensity (up to 4r FLOP/byte) is past
// what the fp32 vector units sustain at 8 TB/s.
#include "common.h"
#include "kernels.h"

namespace lmlp {

namespace {

// ---------------------------------------------------------------------------
// Row projection. Workgroup = 16 token rows x up to 128 output columns; the
// four waves split K (wave w takes k-steps w, w+4, ...), each feeding its own
// accumulators, and the four partial tiles are summed in LDS in fixed order.
// A operand chunks come straight from global memory (one 16-byte load per
// lane per k-step, each 64-byte row segment fully used); the small W factor
// is L2-resident.
template <typename T>
__global__ __launch_bounds__(256) void rowproj_kernel(RowProjParams p) {
  constexpr int CH = elem<T>::CH;
  const RowProjJob& jb = p.job[blockIdx.y];
  const int n_base = blockIdx.z * 128;
  if (n_base >= jb.n1p) return;
  const int nfr = min(8, (jb.n1p - n_base) / 16);
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
  if (t0 >= p.T) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lch = lane >> 4;
  const int64_t row = t0 + lrow;
  const bool rval = row < p.T;
  const T* X = static_cast<const T*>(jb.x) + (rval ? row : 0) * jb.ldx;
  const T* W = static_cast<const T*>(jb.w) + static_cast<int64_t>(n_base + lrow) * jb.ldw;
  const int64_t nchunks = jb.K / CH;
  const int64_t nsteps = (nchunks + 3) / 4;

  f32x4_t acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
  for (int64_t s = wave; s < nsteps; s += 4) {
    const int64_t c = s * 4 + lch;
    const bool cval = c < nchunks;
    const uint4 a = (rval && cval) ? *reinterpret_cast<const uint4*>(X + c * CH) : zero4();
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfr) {
        const uint4 b = cval ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(f) * 16 * jb.ldw + c * CH)
                             : zero4();
        acc[f] = mma<T>::step(b, a, acc[f]);
      }
    }
  }

  __shared__ f32x4_t red[4][8][64];
#pragma unroll
  for (int f = 0; f < 8; ++f)
    if (f < nfr) red[wave][f][lane] = acc[f];
  __syncthreads();
  for (int f = wave; f < nfr; f += 4) {
    f32x4_t v = red[0][f][lane];
    v += red[1][f][lane];
    v += red[2][f][lane];
    v += red[3][f][lane];
    if (!rval) continue;
    // lane holds columns n .. n+3 of token row `row`
    const int n = jb.col_off + n_base + f * 16 + 4 * lch;
    if (jb.out_f32)
      *reinterpret_cast<float4*>(jb.out_f32 + row * jb.ld_f32 + n) = make_float4(v[0], v[1], v[2], v[3]);
    if (jb.out_c) {
      T* o = static_cast<T*>(jb.out_c) + row * jb.ld_c + n;
      store4(o, jb.scale * v[0], jb.scale * v[1], jb.scale * v[2], jb.scale * v[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Column projection. Workgroup = 64 columns k of X (16 per wave) x up to 64
// columns n of P, over one block of tokens, in steps of 32 tokens staged in
// LDS. The MFMA contraction runs over tokens: the P operand is stored
// transposed ([n][t], 16-byte reads) and the X operand is gathered down the
// token axis from a padded row-major tile.
template <typename T>
__global__ __launch_bounds__(256) void colproj_kernel(ColProjParams p) {
  constexpr int CH = elem<T>::CH;
  constexpr int EB = elem<T>::BYTES;
  constexpr int TS = 32;                 // tokens per step
  constexpr int XS = 64 + 4;             // X tile row stride (elements)
  constexpr int PS = TS + 16 / EB;       // P^T tile row stride (elements)
  const ColProjJob& jb = p.job[blockIdx.z];
  const int nblocks = jb.kblocks * jb.ntb * jb.nchunks;
  if (static_cast<int>(blockIdx.x) >= nblocks) return;
  int b = blockIdx.x;
  const int kb = b % jb.kblocks;
  b /= jb.kblocks;
  const int nc = b % jb.nchunks;
  const int tb = b / jb.nchunks;
  const int64_t k0 = static_cast<int64_t>(kb) * 64;
  const int n0 = nc * 64;
  const int nfr = min(4, (jb.n2p - n0) / 16);
  const int64_t tbeg = static_cast<int64_t>(tb) * jb.tr;
  const int64_t tend = min(p.T, tbeg + jb.tr);

  __shared__ __attribute__((aligned(16))) T xs[TS][XS];
  __shared__ __attribute__((aligned(16))) T ps[64][PS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lch = lane >> 4;
  const T* X = static_cast<const T*>(jb.x);

  f32x4_t acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t t = tbeg; t < tend; t += TS) {
    __syncthreads();  // previous step's reads are done
    // X tile: TS rows x 64 elements = TS * (64 / CH) chunks
    constexpr int XCH = 64 / CH;
#pragma unroll
    for (int i = 0; i < (TS * XCH) / 256; ++i) {
      const int q = tid + 256 * i;
      const int r = q / XCH, c = q % XCH;
      const int64_t tt = t + r, kk = k0 + c * CH;
      uint4 v = zero4();
      if (tt < tend && kk < jb.K) v = *reinterpret_cast<const uint4*>(X + tt * jb.ldx + kk);
      uint2* dst = reinterpret_cast<uint2*>(&xs[r][c * CH]);
      dst[0] = make_uint2(v.x, v.y);
      dst[1] = make_uint2(v.z, v.w);
    }
    // P tile: TS rows x 64 fp32, written transposed in the compute dtype
#pragma unroll
    for (int i = 0; i < (TS * 16) / 256; ++i) {
      const int q = tid + 256 * i;
      const int r = q / 16, c4 = (q % 16) * 4;
      const int64_t tt = t + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tt < tend && n0 + c4 < jb.n2p) v = *reinterpret_cast<const float4*>(jb.p + tt * jb.ldp + n0 + c4);
      elem<T>::store(&ps[c4 + 0][r], v.x);
      elem<T>::store(&ps[c4 + 1][r], v.y);
      elem<T>::store(&ps[c4 + 2][r], v.z);
      elem<T>::store(&ps[c4 + 3][r], v.w);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TS / (4 * CH); ++ks) {
      const int tc = ks * 4 + lch;  // token chunk
      const int kl = wave * 16 + lrow;
      uint4 xb;
      if (CH == 8) {
        const uint16_t* base = reinterpret_cast<const uint16_t*>(&xs[0][0]);
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = base[(tc * 8 + e) * XS + kl];
        xb = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      } else {
        const uint32_t* base = reinterpret_cast<const uint32_t*>(&xs[0][0]);
        xb = make_uint4(base[(tc * 4 + 0) * XS + kl], base[(tc * 4 + 1) * XS + kl],
                        base[(tc * 4 + 2) * XS + kl], base[(tc * 4 + 3) * XS + kl]);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (f < nfr) {
          const uint4 pa = *reinterpret_cast<const uint4*>(&ps[f * 16 + lrow][tc * CH]);
          acc[f] = mma<T>::step(pa, xb, acc[f]);
        }
      }
    }
  }
  // lane holds n = n0 + 16f + 4*lch + i for column k = k0 + 16*wave + lrow
  const int64_t k = k0 + wave * 16 + lrow;
  if (k < jb.K) {
    float* out = jb.part + (static_cast<int64_t>(tb) * jb.K + k) * jb.n2p + n0 + 4 * lch;
#pragma unroll
    for (int f = 0; f < 4; ++f)
      if (f < nfr) *reinterpret_cast<float4*>(out + f * 16) = make_float4(acc[f][0], acc[f][1], acc[f][2], acc[f][3]);
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) {
  const ReduceJob& jb = p.job[blockIdx.y];
  const int64_t n = jb.rows * jb.cols;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    int64_t i, j;
    if (jb.transpose) { i = idx % jb.rows; j = idx / jb.rows; }   // consecutive dst columns
    else { j = idx % jb.cols; i = idx / jb.cols; }
    const float* s = jb.src + i * jb.ld_src + jb.col_off + j;
    float v = 0.f;
    for (int c = 0; c < jb.nchunk; ++c) v += s[static_cast<int64_t>(c) * jb.chunk_stride];
    v *= jb.scale;
    const int64_t o = jb.transpose ? j * jb.ld_dst + i : i * jb.ld_dst + j;
    if (jb.dst_bf16) static_cast<uint16_t*>(jb.dst)[o] = f32_to_bf16(v);
    else static_cast<float*>(jb.dst)[o] = v;
  }
}

// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void pack_kernel(PackParams p) {
  const PackJob& jb = p.job[blockIdx.y];
  const int64_t n = jb.rows * jb.cols;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t i = idx / jb.cols, j = idx % jb.cols;
    const int64_t si = jb.transpose ? j : i, sj = jb.transpose ? i : j;
    E v = 0;
    if (jb.src && si < jb.srows && sj < jb.scols) v = static_cast<const E*>(jb.src)[si * jb.ld_src + sj];
    static_cast<E*>(jb.dst)[i * jb.ld_dst + j] = v;
  }
}

// ---------------------------------------------------------------------------
// 8 codes (4 bytes) -> 8 bf16 (16 bytes) per thread iteration
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint8_t* packed, const __half* scales,
                                                           int64_t out, int64_t in, uint4* w) {
  const int64_t n8 = out * in / 8;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n8;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = idx / (in / 8), c = idx % (in / 8);
    const uint32_t q = *reinterpret_cast<const uint32_t*>(packed + row * (in / 2) + c * 4);
    const float sc = __half2float(scales[row * (in / 64) + (c * 8) / 64]);
    w[idx] = dq_chunk(q, sc);
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65535) g = 65535;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_rowproj(const RowProjParams& p, int dtype_bf16, hipStream_t stream) {
  if (p.T <= 0 || p.njobs <= 0) return hipSuccess;
  int maxn = 0;
  for (int i = 0; i < p.njobs; ++i) maxn = p.job[i].n1p > maxn ? p.job[i].n1p : maxn;
  dim3 grid(static_cast<unsigned>((p.T + 15) / 16), p.njobs, (maxn + 127) / 128);
  if (dtype_bf16) hipLaunchKernelGGL(rowproj_kernel<bf16_t>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(rowproj_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_colproj(const ColProjParams& p, int dtype_bf16, hipStream_t stream) {
  if (p.T <= 0 || p.njobs <= 0) return hipSuccess;
  int maxb = 0;
  for (int i = 0; i < p.njobs; ++i) {
    const int nb = p.job[i].kblocks * p.job[i].ntb * p.job[i].nchunks;
    maxb = nb > maxb ? nb : maxb;
  }
  if (maxb == 0) return hipSuccess;
  dim3 grid(maxb, 1, p.njobs);
  if (dtype_bf16) hipLaunchKernelGGL(colproj_kernel<bf16_t>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(colproj_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  if (p.njobs <= 0) return hipSuccess;
  int64_t maxn = 0;
  for (int i = 0; i < p.njobs; ++i) maxn = p.job[i].rows * p.job[i].cols > maxn ? p.job[i].rows * p.job[i].cols : maxn;
  if (maxn == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_kernel, dim3(grid_for(maxn), p.njobs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_pack(const PackParams& p, int elem_bytes, hipStream_t stream) {
  if (p.njobs <= 0) return hipSuccess;
  int64_t maxn = 0;
  for (int i = 0; i < p.njobs; ++i) maxn = p.job[i].rows * p.job[i].cols > maxn ? p.job[i].rows * p.job[i].cols : maxn;
  if (maxn == 0) return hipSuccess;
  dim3 grid(grid_for(maxn), p.njobs);
  if (elem_bytes == 2) hipLaunchKernelGGL(pack_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(pack_kernel<uint32_t>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dequant_int4(const void* packed, const void* scales, int64_t out, int64_t in,
                               void* w_bf16, hipStream_t stream) {
  const int64_t n8 = out * in / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_int4_kernel, dim3(grid_for(n8)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(packed), static_cast<const __half*>(scales), out, in,
                     static_cast<uint4*>(w_bf16));
  return hipGetLastError();
}

}  // namespace lmlp
