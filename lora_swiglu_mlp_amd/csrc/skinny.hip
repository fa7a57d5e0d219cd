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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace lmlp {

namespace {

// ---------------------------------------------------------------------------
// Row projection, fp32, split along K. Workgroup = 256 token rows (64 per
// wave, four MFMA row tiles) x one K slice x up to 64 output columns (four
// MFMA column tiles). Each wave issues the loads of four k-steps (16
// activation chunks and the matching factor chunks) before their MFMAs; each
// factor chunk feeds four row tiles. The slice partials are summed in fixed
// order by proj_finish_kernel. (bf16 uses rowproj_dma_kernel below.)
// job i of a launch: from the kernel arguments, or from the device job table
// when the launch carries more jobs than they hold (a uniform branch). Every
// lane reads the same job; its words are made scalar so that buffer
// descriptors built from it stay in SGPRs.
template <typename J, typename P>
__device__ __forceinline__ J job_at(const P& p, int i) {
  static_assert(sizeof(J) % 4 == 0, "job words");
  J j;
  if (p.table) j = p.table[i];
  else j = p.job[i];
  uint32_t w[sizeof(J) / 4];
  __builtin_memcpy(w, &j, sizeof(J));
#pragma unroll
  for (int k = 0; k < int(sizeof(J) / 4); ++k) w[k] = __builtin_amdgcn_readfirstlane(w[k]);
  __builtin_memcpy(&j, w, sizeof(J));
  return j;
}

constexpr int RP_ROWS = 256;  // token rows per workgroup
template <typename T>
__global__ __launch_bounds__(256) void rowproj_kernel(RowProjParams p) {
  constexpr int CH = elem<T>::CH;
  constexpr int KSTEP = 4 * CH;  // elements per MFMA k-step
  const RowProjJob jb = job_at<RowProjJob>(p, blockIdx.z / p.nsl);
  const int n_base = (blockIdx.z % p.nsl) * 64;
  if (n_base >= jb.n1p || static_cast<int>(blockIdx.y) >= jb.kslices) return;
  if (static_cast<int64_t>(blockIdx.x) * RP_ROWS >= jb.T) return;
  const int nfr = min(4, (jb.n1p - n_base) / 16);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane & 15, lch = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * RP_ROWS + wave * 64 + lrow;  // row tile 0 of this lane
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * jb.kb;
  const int64_t k1 = min(jb.K, k0 + jb.kb);
  const T* X[4];
  bool rval[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = row0 + 16 * r;
    rval[r] = row < jb.T;
    X[r] = static_cast<const T*>(jb.x) + (rval[r] ? row : 0) * jb.ldx;
  }
  const T* W = static_cast<const T*>(jb.w) + static_cast<int64_t>(n_base + lrow) * jb.ldw;

  f32x4_t acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[r][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t kk = k0; kk < k1; kk += 4 * KSTEP) {
    uint4 a[4][4], b[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t c = kk + s * KSTEP + lch * CH;  // first element of this lane's chunk
      const bool cval = c < k1;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[s][r] = (rval[r] && cval) ? *reinterpret_cast<const uint4*>(X[r] + c) : zero4();
#pragma unroll
      for (int f = 0; f < 4; ++f)
        b[s][f] = (f < nfr && cval) ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(f) * 16 * jb.ldw + c)
                                    : zero4();
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int f = 0; f < 4; ++f)
          if (f < nfr) acc[r][f] = mma<T>::step(b[s][f], a[s][r], acc[r][f]);
  }
  // lane holds columns n_base + 16f + 4*lch .. +3 of token row row0 + 16r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!rval[r]) continue;
    float* out = jb.part + (static_cast<int64_t>(blockIdx.y) * jb.T + row0 + 16 * r) * jb.n1p + n_base + 4 * lch;
#pragma unroll
    for (int f = 0; f < 4; ++f)
      if (f < nfr)
        *reinterpret_cast<float4*>(out + f * 16) = make_float4(acc[r][f][0], acc[r][f][1], acc[r][f][2], acc[r][f][3]);
  }
}

// Finish of a split-K row projection: v(t, n) = sum of the slice partials in
// slice order. Writes v to out_f32, scale * v in the compute dtype to out_c,
// and v in the compute dtype, transposed and token-contiguous ([n][ldT],
// zero for T <= t < ldT), to outT; each output is optional. Workgroup = one
// wave on 16 tokens x 64 columns; eight partials are loaded before they are
// added (still in slice order), and the transposed write goes through LDS.
template <typename T, bool TALL>
__global__ __launch_bounds__(64) void proj_finish_kernel(ProjFinishParams p) {
  const ProjFinishJob jb = job_at<ProjFinishJob>(p, blockIdx.z);
  const int64_t tmax = jb.outT ? jb.ldT : jb.T;
  if (jb.n1p <= 0 || tmax <= 0) return;
  // the job's tiles of tr tokens x cw columns, grid-strided over blockIdx.x
  // (a merged launch's jobs differ in token count): 16 x 64, or (TALL: a
  // launch with many tiles) 1024 elements, cw = min(64, n1p rounded up to
  // 16), so that a rank-wide job still gives every lane four items
  const int cw = TALL ? min(64, (jb.n1p + 15) / 16 * 16) : 64;
  const int tr = TALL ? 1024 / cw : 16;  // 16 .. 64, divides ldT
  const int64_t ntn = (jb.n1p + cw - 1) / cw;
  const int64_t ntiles = (tmax + tr - 1) / tr * ntn;
  __shared__ float tile[64 * 17];  // [column][token], token pitch tr + 1: cw (tr + 1) <= 1088
  const int lane = threadIdx.x;
  for (int64_t id = blockIdx.x; id < ntiles; id += gridDim.x) {
    const int n0 = static_cast<int>(id % ntn) * cw;
    const int64_t t0 = id / ntn * tr;
    const int nc = min(cw, jb.n1p - n0);  // a multiple of 4
    const int cpr = nc / 4;               // float4 items per token row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int it = lane + 64 * q;
      if (it >= tr * cpr) break;
      const int tl = it / cpr, c = it % cpr;
      const int64_t t = t0 + tl;
      const int n = n0 + 4 * c;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < jb.T) {
        const float* src = jb.part + t * jb.ld_part + n;
        int k = 0;
        for (; k + 8 <= jb.nparts; k += 8) {
          float4 x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            x[e] = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(k + e) * jb.part_stride);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v.x += x[e].x;
            v.y += x[e].y;
            v.z += x[e].z;
            v.w += x[e].w;
          }
        }
        for (; k < jb.nparts; ++k) {
          const float4 x = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(k) * jb.part_stride);
          v.x += x.x;
          v.y += x.y;
          v.z += x.z;
          v.w += x.w;
        }
        if (jb.out_f32) *reinterpret_cast<float4*>(jb.out_f32 + t * jb.ld_f32 + jb.col_off + n) = v;
        if (jb.out_c)
          store4(static_cast<T*>(jb.out_c) + t * jb.ld_c + jb.col_off + n, jb.scale * v.x, jb.scale * v.y,
                 jb.scale * v.z, jb.scale * v.w);
      }
      tile[(4 * c + 0) * (tr + 1) + tl] = v.x;
      tile[(4 * c + 1) * (tr + 1) + tl] = v.y;
      tile[(4 * c + 2) * (tr + 1) + tl] = v.z;
      tile[(4 * c + 3) * (tr + 1) + tl] = v.w;
    }
    if (!jb.outT) continue;  // uniform over the workgroup
    __syncthreads();
    if (!TALL) {
      if (lane < nc) {  // t0 + 16 <= ldT: ldT is a multiple of 64
        T* dst = static_cast<T*>(jb.outT) + static_cast<int64_t>(jb.col_off + n0 + lane) * jb.ldT + t0;
        const float* src = tile + lane * 17;
#pragma unroll
        for (int e = 0; e < 16; e += 4) store4(dst + e, src[e], src[e + 1], src[e + 2], src[e + 3]);
      }
    } else {
      // rows n of the token-contiguous copy, four consecutive tokens per lane
      // (t0 + tr <= ldT: ldT is a multiple of 64)
      for (int e = lane; e < nc * (tr / 4); e += 64) {
        const int nl = e / (tr / 4), tq = 4 * (e % (tr / 4));
        T* dst = static_cast<T*>(jb.outT) + static_cast<int64_t>(jb.col_off + n0 + nl) * jb.ldT + t0 + tq;
        const float* src = tile + nl * (tr + 1) + tq;
        store4(dst, src[0], src[1], src[2], src[3]);
      }
    }
    __syncthreads();  // the next tile overwrites the staging
  }
}

// ---------------------------------------------------------------------------
// Column projection, fp32 activations. Workgroup = 64 columns k of X (16 per wave) x up to 64
// columns n of P, over one block of tokens, in steps of 32 tokens staged in
// LDS. The MFMA contraction runs over tokens: the P operand is stored
// transposed ([n][t], 16-byte reads) and the X operand is gathered down the
// token axis from a padded row-major tile.
template <typename T>
__global__ __launch_bounds__(256) void colproj_f32_kernel(ColProjParams p) {
  constexpr int CH = elem<T>::CH;
  constexpr int EB = elem<T>::BYTES;
  constexpr int TS = 32;                 // tokens per step
  constexpr int XS = 64 + 4;             // X tile row stride (elements)
  constexpr int PS = TS + 16 / EB;       // P^T tile row stride (elements)
  const ColProjJob jb = job_at<ColProjJob>(p, blockIdx.z);
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
  const int64_t tend = min(jb.T, tbeg + jb.tr);

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
// Column projection, bf16 activations. Workgroup = 256 features x one block of
// tokens x up to 128 output columns. The activation streams through an LDS
// ring of [32 tokens][256 features] tiles (LDS DMA, the N-major tile layout
// and swizzle of the GEMM's B operand), together with the matching
// [n][32 tokens] tile of the transposed P operand (token-contiguous rows,
// chunk c of row r at position c ^ ((r >> 2) & 3)). Transposing reads
// (ds_read_b64_tr_b16) make the token axis the MFMA contraction axis. Wave w
// owns features 64w .. 64w + 63 (four 16-feature MFMA tiles). Every vector
// memory access of this kernel is DMA, so the explicit vmcnt waits are exact.
constexpr int CP_TS = 32;                    // tokens per step
constexpr int CP_XT = CP_TS * 256 * 2;       // activation tile, 16 KB
constexpr int CP_PT = 128 * CP_TS * 2;       // P^T tile, up to 128 columns, 8 KB
constexpr int CP_STAGE = CP_XT + CP_PT;
constexpr int CP_STAGES = 3;                 // 72 KB: two workgroups per CU

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short cp_v4i16_t;
typedef __attribute__((address_space(3))) cp_v4i16_t cp_lds_v4i16_t;

struct CpDma {
  const char* xrow;  // activation at (first token of the block, first feature)
  uint32_t ldx_b;    // activation row stride, bytes
  int64_t tleft;     // tokens of the block from the step being fetched on
  rsrc_t rp;         // P^T rows n0 ..
  uint32_t xoff[4], poff[2];
};

template <int PI>
__device__ __forceinline__ void cp_issue(CpDma& d, char* stage, int step, int wave) {
  const int64_t kr = d.tleft - static_cast<int64_t>(step) * CP_TS;
  const uint32_t krows = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
      static_cast<int>(kr >= CP_TS ? CP_TS : (kr > 0 ? kr : 0))));
  const rsrc_t rx = make_rsrc(d.xrow + static_cast<int64_t>(step) * CP_TS * d.ldx_b, krows * d.ldx_b);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(rx, stage + (4 * wave + i) * 1024, d.xoff[i], 0);
  // prefetches past the block's last step read P^T at step 0 (never used):
  // the uniform offset then stays inside the P^T rows
  const uint32_t soff = kr > 0 ? static_cast<uint32_t>(step) * CP_TS * 2 : 0u;
#pragma unroll
  for (int j = 0; j < PI; ++j) dma16(d.rp, stage + CP_XT + (wave + 4 * j) * 1024, d.poff[j], soff);
}

template <int PI>
__global__ __launch_bounds__(256, 2) void colproj_bf16_kernel(ColProjParams p) {
  const ColProjJob jb = job_at<ColProjJob>(p, blockIdx.z);
  const int nblocks = jb.kblocks * jb.ntb * jb.nchunks;
  if (static_cast<int>(blockIdx.x) >= nblocks) return;
  int b = blockIdx.x;
  const int kb = b % jb.kblocks;
  b /= jb.kblocks;
  const int nc = b % jb.nchunks;
  const int tb = b / jb.nchunks;
  const int64_t f0 = static_cast<int64_t>(kb) * 256;
  const int n0 = nc * 128;
  const int nfr = min(8, (jb.n2p - n0) / 16);
  const int64_t tbeg = static_cast<int64_t>(tb) * jb.tr;
  const int64_t tend = min(jb.T, tbeg + jb.tr);
  if (tbeg >= tend) return;
  const int nsteps = static_cast<int>((tend - tbeg + CP_TS - 1) / CP_TS);

  __shared__ __attribute__((aligned(1024))) char ring[CP_STAGES * CP_STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15, lgrp = lane >> 4;

  CpDma d;
  d.ldx_b = static_cast<uint32_t>(jb.ldx * 2);
  d.xrow = static_cast<const char*>(jb.x) + (tbeg * jb.ldx + f0) * 2;
  d.tleft = tend - tbeg;
  const uint32_t ldp_b = static_cast<uint32_t>(jb.ldpT * 2);
  d.rp = make_rsrc(static_cast<const char*>(jb.pT) + static_cast<int64_t>(n0) * jb.ldpT * 2 + tbeg * 2,
                   static_cast<uint32_t>(16 * nfr) * ldp_b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = 2 * (4 * wave + i) + (lane >> 5);
    const int fc = (lane & 31) ^ nn_swz(k);
    d.xoff[i] = (f0 + fc * 8 < jb.K) ? static_cast<uint32_t>(k) * d.ldx_b + fc * 16 : DMA_OOB;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int f = wave + 4 * j;  // P^T row tile of instruction j
    const int rr = lane >> 2;
    const int lc = (lane & 3) ^ ((rr >> 2) & 3);
    d.poff[j] = f < nfr ? static_cast<uint32_t>(16 * f + rr) * ldp_b + lc * 16 : DMA_OOB;
  }

  // fragment read addresses: activation (transposing), P^T (16-byte rows)
  const uint32_t rdN = static_cast<uint32_t>((lgrp * 8 + (lrow >> 2)) * 512 +
                                             ((wave >> 1) * 16 + ((lrow & 3) >> 1)) * 16 + 8 * (lrow & 1));
  const int nsw = 2 * ((lrow >> 2) | ((lgrp & 1) << 2));
  const uint32_t rdP = static_cast<uint32_t>(CP_XT + lrow * 64 + ((lgrp ^ ((lrow >> 2) & 3)) << 4));

  f32x4_t acc[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[j][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  cp_issue<PI>(d, ring, 0, wave);
  cp_issue<PI>(d, ring + CP_STAGE, 1, wave);
  wait_vmcnt<4 + PI>();  // step 0 landed (this wave)
  __syncthreads();
  int cur = 0;
  for (int s = 0; s < nsteps; ++s) {
    const char* st = ring + cur * CP_STAGE;
    const int nx = cur == 0 ? CP_STAGES - 1 : cur - 1;  // stage of step s+2 (step s-1's)
    cp_issue<PI>(d, ring + nx * CP_STAGE, s + 2, wave);
    uint4 xf[4], pf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bb = 4 * (wave & 1) + j;
      const uint32_t base = rdN + ((((2 * bb) ^ nsw) & 15) << 4);
      const cp_v4i16_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((cp_lds_v4i16_t*)(st + base));
      const cp_v4i16_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((cp_lds_v4i16_t*)(st + base + 4 * 512));
      const uint2 u0 = __builtin_bit_cast(uint2, t0);
      const uint2 u1 = __builtin_bit_cast(uint2, t1);
      xf[j] = make_uint4(u0.x, u0.y, u1.x, u1.y);
    }
#pragma unroll
    for (int f = 0; f < 8; ++f)
      if (f < nfr) pf[f] = *reinterpret_cast<const uint4*>(st + rdP + f * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int f = 0; f < 8; ++f)
        if (f < nfr) acc[j][f] = mma<bf16_t>::step(pf[f], xf[j], acc[j][f]);
    wait_vmcnt<4 + PI>();  // step s+1 landed (this wave); step s+2 may still fly
    __syncthreads();       // ... everywhere, and every read of stage `cur` is done
    cur = cur + 1 == CP_STAGES ? 0 : cur + 1;
  }
  wait_vmcnt<0>();  // the prefetches past the last step
  // lane holds n = n0 + 16f + 4*lgrp .. +3 for feature f0 + 64*wave + 16j + lrow
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t feat = f0 + 64 * wave + 16 * j + lrow;
    if (feat >= jb.K) continue;
    float* out = jb.part + (static_cast<int64_t>(tb) * jb.K + feat) * jb.n2p + n0 + 4 * lgrp;
#pragma unroll
    for (int f = 0; f < 8; ++f)
      if (f < nfr)
        *reinterpret_cast<float4*>(out + 16 * f) = make_float4(acc[j][f][0], acc[j][f][1], acc[j][f][2], acc[j][f][3]);
  }
}

// ---------------------------------------------------------------------------
// Fixed-order sum of partials: v(i, j) = scale * sum_c src[c][i][col_off + j]
// for i < rows, j < cols, written to dst[i][j] or, with transpose, dst[j][i],
// in fp32 or bf16. Workgroup = one wave on a 16 x 64 tile or, in a launch
// with many tiles (TALL: a merged launch over many experts), on a tile of
// 1024 elements: CW = min(64, cols rounded up to 16) columns by 1024 / CW
// rows, so a rank-wide job (16 columns) gets 64-row tiles and every lane
// still has its four 16-byte items (with few tiles the 16-row ones keep
// more workgroups busy). Reads are 16 bytes per lane along source rows with eight
// partials in flight (summed in partial order); the transposed case goes
// through LDS so that its writes also run along destination rows. nchunk =
// 0 writes zeros.
template <bool TALL>
__global__ __launch_bounds__(64) void reduce_kernel(ReduceParams p) {
  const ReduceJob jb = job_at<ReduceJob>(p, blockIdx.z);
  if (jb.rows <= 0 || jb.cols <= 0) return;
  const int cw = TALL ? static_cast<int>(min<int64_t>(64, (jb.cols + 15) / 16 * 16)) : 64;  // tile columns
  const int tr = TALL ? 1024 / cw : 16;                                                    // tile rows: 16 .. 64
  // the job's tiles, numbered row-major, grid-strided over blockIdx.x (a
  // merged launch's jobs differ in shape: tall and wide ones)
  const int64_t ntj = (jb.cols + cw - 1) / cw;
  const int64_t ntiles = (jb.rows + tr - 1) / tr * ntj;
  __shared__ float tile[64 * 17];  // [column][row], row pitch tr + 1: cw (tr + 1) <= 1088 for every cw
  const int lane = threadIdx.x;
  for (int64_t id = blockIdx.x; id < ntiles; id += gridDim.x) {
    const int64_t i0 = id / ntj * tr;
    const int64_t j0 = id % ntj * cw;
    const int64_t ncols = min<int64_t>(cw, jb.cols - j0);
    const int cpr = static_cast<int>((ncols + 3) / 4);  // float4 items per source row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int it = lane + 64 * q;
      if (it >= tr * cpr) break;
      const int il = it / cpr, c = it % cpr;
      const int64_t i = i0 + il;
      const int64_t j = j0 + 4 * c;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (i < jb.rows) {
        const float* s = jb.src + i * jb.ld_src + jb.col_off + j;
        int k = 0;
        for (; k + 8 <= jb.nchunk; k += 8) {
          float4 x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            x[e] = *reinterpret_cast<const float4*>(s + static_cast<int64_t>(k + e) * jb.chunk_stride);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[0] += x[e].x;
            v[1] += x[e].y;
            v[2] += x[e].z;
            v[3] += x[e].w;
          }
        }
        for (; k < jb.nchunk; ++k) {
          const float4 x = *reinterpret_cast<const float4*>(s + static_cast<int64_t>(k) * jb.chunk_stride);
          v[0] += x.x;
          v[1] += x.y;
          v[2] += x.z;
          v[3] += x.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= jb.scale;
      if (!jb.transpose) {
        if (i < jb.rows) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (j + e >= jb.cols) break;
            const int64_t o = i * jb.ld_dst + j + e;
            if (jb.dst_bf16) static_cast<uint16_t*>(jb.dst)[o] = f32_to_bf16(v[e]);
            else static_cast<float*>(jb.dst)[o] = v[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[(4 * c + e) * (tr + 1) + il] = v[e];
      }
    }
    if (!jb.transpose) continue;  // uniform over the workgroup
    __syncthreads();
    if (tr == 16) {  // lane j writes its column's 16 rows
      const int64_t j = j0 + lane;
      if (lane < ncols) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t i = i0 + e;
          if (i >= jb.rows) break;
          const int64_t o = j * jb.ld_dst + i;
          const float v = tile[lane * 17 + e];
          if (jb.dst_bf16) static_cast<uint16_t*>(jb.dst)[o] = f32_to_bf16(v);
          else static_cast<float*>(jb.dst)[o] = v;
        }
      }
      __syncthreads();  // the next tile overwrites the staging
      continue;
    }
    // destination rows j (the tile's columns), tr consecutive elements each
    for (int e = lane; e < ncols * tr; e += 64) {
      const int jl = e / tr, il = e % tr;
      const int64_t i = i0 + il;
      if (i >= jb.rows) continue;
      const int64_t o = (j0 + jl) * jb.ld_dst + i;
      const float v = tile[jl * (tr + 1) + il];
      if (jb.dst_bf16) static_cast<uint16_t*>(jb.dst)[o] = f32_to_bf16(v);
      else static_cast<float*>(jb.dst)[o] = v;
    }
    __syncthreads();  // the next tile overwrites the staging
  }
}

// ---------------------------------------------------------------------------
// Zero-padded copy of an adapter factor, dst[i][j] = src[i][j] where the
// source has that element, else 0 (i < rows, j < cols), or with transpose
// dst[i][j] = src[j][i]. Plain copies: a thread moves groups of 16 bytes (G
// consecutive destination elements of one row), four groups in flight per
// iteration, with 16-byte accesses wherever rows and pointers allow.
// Transposes (at most 64 destination rows, the rank): 64 source rows at a
// time through LDS, read along source rows and written along destination
// rows. 32-bit index arithmetic (every factor has far fewer than 2^31
// elements).
template <typename E>
__global__ __launch_bounds__(256) void pack_kernel(PackParams p) {
  __shared__ E tile[64 * 65];
  const PackJob jb = job_at<PackJob>(p, blockIdx.y);
  const uint32_t rows = static_cast<uint32_t>(jb.rows), cols = static_cast<uint32_t>(jb.cols);
  const uint32_t srows = static_cast<uint32_t>(jb.srows), scols = static_cast<uint32_t>(jb.scols);
  const E* src = static_cast<const E*>(jb.src);
  E* dst = static_cast<E*>(jb.dst);
  const uint32_t ld_dst = static_cast<uint32_t>(jb.ld_dst), ld_src = static_cast<uint32_t>(jb.ld_src);
  if (jb.transpose && rows <= 64) {
    for (uint32_t j0 = blockIdx.x * 64; j0 < cols; j0 += gridDim.x * 64) {
      // source rows j0 .. j0 + 63, their first `rows` elements
      for (uint32_t e = threadIdx.x; e < 64 * rows; e += 256) {
        const uint32_t jj = e / rows, i = e % rows, j = j0 + jj;
        E v = 0;
        if (src && j < srows && i < scols && j < cols) v = src[j * ld_src + i];
        tile[jj * 65 + i] = v;
      }
      __syncthreads();
      for (uint32_t e = threadIdx.x; e < rows * 64; e += 256) {
        const uint32_t i = e / 64, jj = e % 64, j = j0 + jj;
        if (j < cols) dst[i * ld_dst + j] = tile[jj * 65 + i];
      }
      __syncthreads();
    }
    return;
  }
  constexpr uint32_t G = 16 / sizeof(E);  // elements per group
  const uint32_t cq = (cols + G - 1) / G;  // groups per destination row
  const uint32_t n = rows * cq;
  const bool vdst = ld_dst % G == 0 && reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  const bool vsrc = src && !jb.transpose && ld_src % G == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0;
  const uint32_t stride = gridDim.x * 256;
  for (uint32_t base = blockIdx.x * 256 + threadIdx.x; base < n; base += 4 * stride) {
    E v[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t idx = base + u * stride;
      const uint32_t i = idx / cq, j0 = (idx % cq) * G;
#pragma unroll
      for (uint32_t e = 0; e < G; ++e) v[u][e] = 0;
      if (idx >= n || !src) continue;
      if (vsrc && i < srows && j0 + G - 1 < scols) {
        const uint4 w = *reinterpret_cast<const uint4*>(src + i * ld_src + j0);
        __builtin_memcpy(v[u], &w, 16);
      } else {
#pragma unroll
        for (uint32_t e = 0; e < G; ++e) {
          const uint32_t j = j0 + e;
          const uint32_t si = jb.transpose ? j : i, sj = jb.transpose ? i : j;
          if (j < cols && si < srows && sj < scols) v[u][e] = src[si * ld_src + sj];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t idx = base + u * stride;
      if (idx >= n) continue;
      const uint32_t i = idx / cq, j0 = (idx % cq) * G;
      E* d = dst + i * ld_dst + j0;
      if (vdst && j0 + G - 1 < cols) {
        uint4 w;
        __builtin_memcpy(&w, v[u], 16);
        *reinterpret_cast<uint4*>(d) = w;
      } else {
#pragma unroll
        for (uint32_t e = 0; e < G; ++e)
          if (j0 + e < cols) d[e] = v[u][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 block scales [rows][nb] -> fp32 [nb][ld_dst] (block-major), so that
// the scales of one k-block of consecutive weight rows are contiguous.
__global__ __launch_bounds__(256) void scale_pack_kernel(ScalePackParams p) {
  const ScalePackJob& jb = p.job[blockIdx.y];
  const int64_t n = jb.rows * jb.nb;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    if (jb.row_major) {
      const int64_t r = idx / jb.nb, b = idx % jb.nb;
      jb.dst[r * jb.ld_dst + b] = __half2float(jb.src[idx]);
    } else {
      const int64_t b = idx / jb.rows, r = idx % jb.rows;
      jb.dst[b * jb.ld_dst + r] = __half2float(jb.src[r * jb.nb + b]);
    }
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

// ---------------------------------------------------------------------------
// Split-K finish: four consecutive outputs per thread, the slices summed in
// slice order, one rounding to bf16.
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ part, int nsplit, int64_t n4,
                                                         int64_t stride, uint2* __restrict__ y) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float4 acc = reinterpret_cast<const float4*>(part)[i];
    for (int s = 1; s < nsplit; ++s) {
      const float4 v = reinterpret_cast<const float4*>(part + s * stride)[i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    y[i] = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65535) g = 65535;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

// ---------------------------------------------------------------------------
// Row projection, bf16, streamed through LDS by DMA. Workgroup = 128 token
// rows (32 per wave, two MFMA row tiles) x one K slice x up to 16*NF output
// columns (NF column tiles, 2 or 4). A ring of NS stages holds, per 64
// elements of K, the activation tile [128 rows][128 bytes] and the factor
// tile [16*NF rows][128 bytes], chunk c of row n at position c ^ (n & 7)
// (whole 128-byte lines per row, conflict-free fragment reads). Each wave
// issues 4 + NF/2 DMA instructions of 1 KB per stage, so NS-1 stages are in
// flight per workgroup with no registers held; two workgroups share a CU.
// Rows past T and K past the slice read zero.
constexpr int RPD_ROWS = 128;
constexpr int RPD_BK = 64;               // K elements per stage
constexpr int RPD_XT = RPD_ROWS * 128;   // activation tile bytes

template <int NF, int NS>
__global__ __launch_bounds__(256, 2) void rowproj_dma_kernel(RowProjParams p) {
  constexpr int STAGE = RPD_XT + 16 * NF * 128;
  constexpr int NW = NF / 2;  // factor DMA instructions per wave and stage
  const RowProjJob jb = job_at<RowProjJob>(p, blockIdx.z / p.nsl);
  const int n_base = (blockIdx.z % p.nsl) * 16 * NF;
  if (n_base >= jb.n1p || static_cast<int>(blockIdx.y) >= jb.kslices) return;
  const int nfr = min(NF, (jb.n1p - n_base) / 16);
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * jb.kb;
  const int64_t k1 = min(jb.K, k0 + jb.kb);
  if (k0 >= k1) return;
  const int nst = static_cast<int>((k1 - k0 + RPD_BK - 1) / RPD_BK);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * RPD_ROWS;
  if (r0 >= jb.T) return;  // a job with fewer rows than the launch's widest

  __shared__ __attribute__((aligned(1024))) char ring[NS * STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15, lch = lane >> 4;

  // DMA pattern: activation instruction i of this wave fills rows
  // 32*wave + 8*i + lane/8, factor instruction j rows 8*(NW*wave + j) + lane/8;
  // position lane & 7 holds chunk (lane & 7) ^ (row & 7)
  const uint32_t ldx_b = static_cast<uint32_t>(jb.ldx * 2), ldw_b = static_cast<uint32_t>(jb.ldw * 2);
  const rsrc_t rx = make_rsrc(static_cast<const char*>(jb.x) + r0 * ldx_b,
                              static_cast<uint32_t>(min<int64_t>(RPD_ROWS, jb.T - r0)) * ldx_b);
  const rsrc_t rw = make_rsrc(static_cast<const char*>(jb.w) + static_cast<int64_t>(n_base) * ldw_b,
                              static_cast<uint32_t>(16 * nfr) * ldw_b);
  uint32_t xo[4], wo[NW];
  int xc[4], wc[NW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    xc[i] = (lane & 7) ^ (row & 7);
    xo[i] = r0 + row < jb.T ? static_cast<uint32_t>(row) * ldx_b + xc[i] * 16 : DMA_OOB;
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int row = 8 * (NW * wave + j) + (lane >> 3);
    wc[j] = (lane & 7) ^ (row & 7);
    wo[j] = row < 16 * nfr ? static_cast<uint32_t>(row) * ldw_b + wc[j] * 16 : DMA_OOB;
  }
  // stage s of the slice (past the last one: all lanes out of range, so the
  // wait counts stay uniform)
  auto issue = [&](int s) {
    char* st = ring + (s % NS) * STAGE;
    const int64_t k = k0 + static_cast<int64_t>(s) * RPD_BK;
    const bool live = s < nst;
    const uint32_t soff = live ? static_cast<uint32_t>(k * 2) : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(rx, st + (32 * wave + 8 * i) * 128, (live && k + xc[i] * 8 < k1) ? xo[i] : DMA_OOB, soff);
#pragma unroll
    for (int j = 0; j < NW; ++j)
      dma16(rw, st + RPD_XT + 8 * (NW * wave + j) * 128, (live && k + wc[j] * 8 < k1) ? wo[j] : DMA_OOB, soff);
  };

  f32x4_t acc[2][NF];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[r][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  for (int s = 0; s < nst; ++s) {
    wait_vmcnt<(4 + NW) * (NS - 2)>();  // stage s landed (this wave)
    __syncthreads();                    // ... everywhere; stage s-1 is free
    issue(s + NS - 1);
    const char* st = ring + (s % NS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 4 * ks + lch;
      uint4 xf[2], wf[NF];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 32 * wave + 16 * r + lrow;
        xf[r] = *reinterpret_cast<const uint4*>(st + row * 128 + ((ch ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int row = 16 * f + lrow;
        if (f < nfr) wf[f] = *reinterpret_cast<const uint4*>(st + RPD_XT + row * 128 + ((ch ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (f < nfr) acc[r][f] = mma<bf16_t>::step(wf[f], xf[r], acc[r][f]);
    }
  }
  wait_vmcnt<0>();  // the stages issued past the last one
  // lane holds columns n_base + 16f + 4*lch .. +3 of token row r0 + 32*wave + 16r + lrow
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int64_t row = r0 + 32 * wave + 16 * r + lrow;
    if (row >= jb.T) continue;
    float* out = jb.part + (static_cast<int64_t>(blockIdx.y) * jb.T + row) * jb.n1p + n_base + 4 * lch;
#pragma unroll
    for (int f = 0; f < NF; ++f)
      if (f < nfr)
        *reinterpret_cast<float4*>(out + f * 16) = make_float4(acc[r][f][0], acc[r][f][1], acc[r][f][2], acc[r][f][3]);
  }
}

}  // namespace

hipError_t launch_rowproj(const RowProjParams& p, int dtype_bf16, hipStream_t stream, const RowProjJob* hjobs) {
  if (p.T <= 0 || p.njobs <= 0) return hipSuccess;
  if ((hjobs != nullptr) != (p.table != nullptr) || (!hjobs && p.njobs > 52)) return hipErrorInvalidValue;
  RowProjParams q = p;
  if (!hjobs)
    for (int i = 0; i < q.njobs; ++i)
      if (q.job[i].T == 0) q.job[i].T = q.T;
  const RowProjJob* js = hjobs ? hjobs : q.job;
  int maxn = 0, maxks = 0;
  for (int i = 0; i < q.njobs; ++i) {
    maxn = js[i].n1p > maxn ? js[i].n1p : maxn;
    maxks = js[i].kslices > maxks ? js[i].kslices : maxks;
  }
  if (maxks == 0 || maxn == 0) return hipSuccess;
  if (q.njobs * static_cast<int64_t>((maxn + 31) / 32) > 65535) return hipErrorInvalidValue;  // grid.z
  if (dtype_bf16) {
    const bool wide = maxn > 32;  // 64 columns a pass (4 stages of 24 KB would not fit twice)
    q.nsl = wide ? (maxn + 63) / 64 : (maxn + 31) / 32;
    dim3 grid(static_cast<unsigned>((q.T + RPD_ROWS - 1) / RPD_ROWS), maxks, q.njobs * q.nsl);
    if (wide) hipLaunchKernelGGL((rowproj_dma_kernel<4, 3>), grid, dim3(256), 0, stream, q);
    else hipLaunchKernelGGL((rowproj_dma_kernel<2, 4>), grid, dim3(256), 0, stream, q);
  } else {
    q.nsl = (maxn + 63) / 64;
    dim3 grid(static_cast<unsigned>((q.T + RP_ROWS - 1) / RP_ROWS), maxks, q.njobs * q.nsl);
    hipLaunchKernelGGL(rowproj_kernel<float>, grid, dim3(256), 0, stream, q);
  }
  return hipGetLastError();
}

hipError_t launch_proj_finish(const ProjFinishParams& p0, int dtype_bf16, hipStream_t stream,
                              const ProjFinishJob* hjobs) {
  if (p0.njobs <= 0) return hipSuccess;
  if ((hjobs != nullptr) != (p0.table != nullptr) || (!hjobs && p0.njobs > 36) || p0.njobs > 65535)
    return hipErrorInvalidValue;
  ProjFinishParams p = p0;
  if (!hjobs)
    for (int i = 0; i < p.njobs; ++i)
      if (p.job[i].T == 0) p.job[i].T = p.T;
  const ProjFinishJob* js = hjobs ? hjobs : p.job;
  // 16 x 64 tiles in all; past 1024 of them, narrow jobs go in taller tiles
  int64_t all = 0;
  for (int i = 0; i < p.njobs; ++i) {
    const int64_t t = js[i].outT ? js[i].ldT : js[i].T;
    all += (t + 15) / 16 * ((js[i].n1p + 63) / 64);
  }
  p.tall = all > 1024 ? 1 : 0;
  int64_t maxtiles = 0;  // tiles of the largest job, as the kernel cuts them
  for (int i = 0; i < p.njobs; ++i) {
    const int64_t t = js[i].outT ? js[i].ldT : js[i].T;
    if (js[i].n1p <= 0 || t <= 0) continue;
    const int64_t cw = p.tall ? std::min<int64_t>(64, (js[i].n1p + 15) / 16 * 16) : 64;
    const int64_t nt = (t + 1024 / cw - 1) / (1024 / cw) * ((js[i].n1p + cw - 1) / cw);
    maxtiles = nt > maxtiles ? nt : maxtiles;
  }
  if (maxtiles <= 0) return hipSuccess;
  // about 16 K workgroups in all; each strides over its job's tiles
  dim3 grid(static_cast<unsigned>(std::min<int64_t>(maxtiles, std::max<int64_t>(1, 16384 / p.njobs))), 1, p.njobs);
  if (dtype_bf16) {
    if (p.tall) hipLaunchKernelGGL((proj_finish_kernel<bf16_t, true>), grid, dim3(64), 0, stream, p);
    else hipLaunchKernelGGL((proj_finish_kernel<bf16_t, false>), grid, dim3(64), 0, stream, p);
  } else {
    if (p.tall) hipLaunchKernelGGL((proj_finish_kernel<float, true>), grid, dim3(64), 0, stream, p);
    else hipLaunchKernelGGL((proj_finish_kernel<float, false>), grid, dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_colproj(const ColProjParams& p0, int dtype_bf16, hipStream_t stream, const ColProjJob* hjobs) {
  if (p0.T <= 0 || p0.njobs <= 0) return hipSuccess;
  if ((hjobs != nullptr) != (p0.table != nullptr) || (!hjobs && p0.njobs > 38) || p0.njobs > 65535)
    return hipErrorInvalidValue;
  ColProjParams p = p0;
  if (!hjobs)
    for (int i = 0; i < p.njobs; ++i)
      if (p.job[i].T == 0) p.job[i].T = p.T;
  const ColProjJob* js = hjobs ? hjobs : p.job;
  int maxb = 0, maxfr = 0;
  for (int i = 0; i < p.njobs; ++i) {
    const ColProjJob& j = js[i];
    const int nb = j.kblocks * j.ntb * j.nchunks;
    maxb = nb > maxb ? nb : maxb;
    const int fr = (j.n2p < 128 ? j.n2p : 128) / 16;
    maxfr = fr > maxfr ? fr : maxfr;
  }
  if (maxb == 0) return hipSuccess;
  dim3 grid(maxb, 1, p.njobs);
  if (!dtype_bf16) hipLaunchKernelGGL(colproj_f32_kernel<float>, grid, dim3(256), 0, stream, p);
  else if (maxfr <= 4) hipLaunchKernelGGL(colproj_bf16_kernel<1>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(colproj_bf16_kernel<2>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream, const ReduceJob* hjobs) {
  if (p.njobs <= 0) return hipSuccess;
  if ((hjobs != nullptr) != (p.table != nullptr) || (!hjobs && p.njobs > 46) || p.njobs > 65535)
    return hipErrorInvalidValue;
  const ReduceJob* js = hjobs ? hjobs : p.job;
  // 16 x 64 tiles in all; past 8192 of them, rank-wide jobs go in taller tiles
  int64_t all = 0;
  for (int i = 0; i < p.njobs; ++i) all += (js[i].rows + 15) / 16 * ((js[i].cols + 63) / 64);
  ReduceParams q = p;
  q.tall = all > 8192 ? 1 : 0;
  int64_t maxt = 0;  // tiles of the largest job, as the kernel cuts them
  for (int i = 0; i < p.njobs; ++i) {
    if (js[i].rows <= 0 || js[i].cols <= 0) continue;
    const int64_t cw = q.tall ? std::min<int64_t>(64, (js[i].cols + 15) / 16 * 16) : 64;
    const int64_t t = (js[i].rows + 1024 / cw - 1) / (1024 / cw) * ((js[i].cols + cw - 1) / cw);
    maxt = t > maxt ? t : maxt;
  }
  if (maxt == 0) return hipSuccess;
  // about 16 K workgroups in all; each strides over its job's tiles
  const int64_t cap = std::max<int64_t>(1, 16384 / p.njobs);
  dim3 grid(static_cast<unsigned>(std::min<int64_t>(maxt, cap)), 1, p.njobs);
  if (q.tall) hipLaunchKernelGGL(reduce_kernel<true>, grid, dim3(64), 0, stream, q);
  else hipLaunchKernelGGL(reduce_kernel<false>, grid, dim3(64), 0, stream, q);
  return hipGetLastError();
}

hipError_t launch_pack(const PackParams& p, int elem_bytes, hipStream_t stream, const PackJob* hjobs) {
  if (p.njobs <= 0) return hipSuccess;
  if ((hjobs != nullptr) != (p.table != nullptr) || (!hjobs && p.njobs > 52) || p.njobs > 65535)
    return hipErrorInvalidValue;
  const PackJob* js = hjobs ? hjobs : p.job;
  int64_t maxn = 0;
  for (int i = 0; i < p.njobs; ++i) maxn = js[i].rows * js[i].cols > maxn ? js[i].rows * js[i].cols : maxn;
  if (maxn == 0) return hipSuccess;
  if (elem_bytes != 2 && elem_bytes != 4) return hipErrorInvalidValue;
  // plain copies in one pass of their workgroups (four groups of 16 bytes
  // per thread), transposes one 64-column tile per workgroup; a merged
  // launch's grid is as wide as its widest job, so when that leaves over
  // 8192 workgroups (many experts' jobs) transposes take four tiles per
  // workgroup: fewer, fuller workgroups, fewer idle ones for the small jobs
  int64_t maxg = 1;
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t per = pass == 0 ? 64 : 256;  // columns per transposing workgroup
    maxg = 1;
    for (int i = 0; i < p.njobs; ++i) {
      const int64_t g = js[i].transpose && js[i].rows <= 64
                            ? (js[i].cols + per - 1) / per
                            : (js[i].rows * ((js[i].cols * elem_bytes + 15) / 16) + 1023) / 1024;
      maxg = g > maxg ? g : maxg;
    }
    if (maxg * p.njobs <= 8192) break;
  }
  dim3 grid(static_cast<unsigned>(std::min<int64_t>(maxg, 65535)), p.njobs);
  if (elem_bytes == 2) hipLaunchKernelGGL(pack_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(pack_kernel<uint32_t>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_splitk_sum(const float* part, int nsplit, int64_t n, void* y_bf16, hipStream_t stream) {
  if (nsplit < 1 || n % 4) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const int64_t n4 = n / 4;
  int64_t g = (n4 + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(splitk_sum_kernel, dim3(static_cast<int>(g)), dim3(256), 0, stream, part, nsplit, n4, n,
                     static_cast<uint2*>(y_bf16));
  return hipGetLastError();
}

hipError_t launch_scale_pack(const ScalePackParams& p, hipStream_t stream) {
  if (p.njobs <= 0) return hipSuccess;
  int64_t maxn = 0;
  for (int i = 0; i < p.njobs; ++i) maxn = p.job[i].rows * p.job[i].nb > maxn ? p.job[i].rows * p.job[i].nb : maxn;
  if (maxn == 0) return hipSuccess;
  hipLaunchKernelGGL(scale_pack_kernel, dim3(grid_for(maxn), p.njobs), dim3(256), 0, stream, p);
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
