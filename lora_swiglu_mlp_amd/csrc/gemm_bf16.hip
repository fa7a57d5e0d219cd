// bf16 MFMA GEMM for gfx950 with LDS-DMA operand staging.
//
// Same products, K segments and epilogues as the general kernel in gemm.hip
// (base K loop plus the appended rank-r adapter K-steps of the fused LoRA MLP,
// "Unsloth 深度分析报告", section 创新之处), specialised for dense bf16:
//
//  * Operands go global -> LDS with buffer_load ... lds (16 bytes per lane),
//    so no VGPRs hold staged tiles and no VALU moves data. Each instruction
//    writes 1 KB of LDS linearly; the XOR swizzle is applied by choosing which
//    global chunk each lane fetches. Out-of-range rows, columns and K tails
//    read as zero through the buffer range check (the offset of an invalid
//    chunk is set past the range), so the loop has no branches.
//  * K-major operands (A always, B in the NT products) sit in LDS as
//    [256 rows][128 bytes]; the MFMA operand reads are 16-byte ds_read_b128.
//  * N-major B operands (the NN products dZ = dY W_d and dX = dG W_g + dU W_u)
//    sit in LDS exactly as in memory, [64 k][256 n], and are transposed on the
//    way to registers by ds_read_b64_tr_b16: within each 16-lane group, lane j
//    names 4 consecutive n of row k0 + j/4, and lane i receives column i of
//    the four rows, i.e. 4 consecutive k of one n (the MFMA operand layout).
//  * Two LDS stages of 64 KB: the DMA for tile k+1 is issued right after the
//    barrier that opens tile k and runs under tile k's 128 MFMAs per wave.
#include "common.h"
#include "gemm_epilogue.h"
#include "kernels.h"

#ifndef LMLP_SCHED_FENCES
#define LMLP_SCHED_FENCES 1
#endif
#if LMLP_SCHED_FENCES
#define LMLP_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define LMLP_SCHED_FENCE() ((void)0)
#endif

namespace lmlp {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;              // bf16 elements of K per tile (128 bytes)
constexpr int NTHREADS = 256;
constexpr int TILE_BYTES = 32768;   // one operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr uint32_t OOB = 0x80000000u;  // buffer offset that fails the range check

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4i16_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(nbytes), 0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds_dst), 16,
                                           static_cast<int>(voff), 0, 0, 0);
}

// swizzle of 16-byte chunk positions in an N-major [k][256 n] tile row:
// the rows one transposing read touches (4 consecutive k, and k + 8) map a
// pair of chunks to 8 distinct pairs of bank groups
__device__ __forceinline__ int nn_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

// one K segment of the product (all values uniform)
struct Seg {
  const char* a;
  const char* b0;
  const char* b1;
  uint32_t lda_b, ldb_b;  // row strides in bytes
  int K;                  // elements
};

__device__ __forceinline__ Seg seg_at(const GemmParams& p, int s) {
  const GemmSeg& g = p.seg[s];
  Seg d;
  d.a = static_cast<const char*>(g.a);
  d.b0 = static_cast<const char*>(g.b0);
  d.b1 = static_cast<const char*>(g.b1);
  d.lda_b = static_cast<uint32_t>(g.lda * 2);
  d.ldb_b = static_cast<uint32_t>(g.ldb * 2);
  d.K = s < p.nseg ? static_cast<int>(g.K) : 0;
  return d;
}

__device__ __forceinline__ Seg seg_pick(int sg, const Seg& s0, const Seg& s1, const Seg& s2) {
  Seg d;
  d.a = sg == 0 ? s0.a : (sg == 1 ? s1.a : s2.a);
  d.b0 = sg == 0 ? s0.b0 : (sg == 1 ? s1.b0 : s2.b0);
  d.b1 = sg == 0 ? s0.b1 : (sg == 1 ? s1.b1 : s2.b1);
  d.lda_b = sg == 0 ? s0.lda_b : (sg == 1 ? s1.lda_b : s2.lda_b);
  d.ldb_b = sg == 0 ? s0.ldb_b : (sg == 1 ? s1.ldb_b : s2.ldb_b);
  d.K = sg == 0 ? s0.K : (sg == 1 ? s1.K : s2.K);
  return d;
}

// where this workgroup's output tile sits, and the lane's roles
struct TileCtx {
  int64_t m0, n0, j0;     // j0: first gate/up column (n0 / 2)
  uint32_t m_rows, n_rows;
  int64_t N;
  int wave, lane, c0;     // c0 = (lane & 7) ^ (lane >> 3)
};

// DMA state of the tile fetched next
struct Dma {
  __amdgpu_buffer_rsrc_t rA, rB0, rB1;
  uint32_t offA[8], offB[8];
  Seg S;
  int seg, k0, kt;
};

// Per-lane offsets of the DMA pattern for segment S.
// K-major tiles: instruction i of this wave fills tile rows
// 64*wave + 8*i + (lane >> 3), chunk position lane & 7; with row & 7 ==
// lane >> 3 and (row >> 3) & 7 == i (mod 8) the logical chunk swz(row, lane&7)
// there is c0 ^ i. Gate/up B operand: tile rows alternate gate/up every 16,
// so instruction i reads weight row (2*wave + i/4)*16 + 8*(i&1) + lane/8 of
// the gate (i&2 == 0) or up panel. N-major B tiles: instruction i fills rows
// k = 2*(8*wave + i) + (lane >> 5), chunk position lane & 31 holding n-chunk
// (lane & 31) ^ nn_swz(k); chunks past N are never fetched.
template <bool NN, int EPI>
__device__ __forceinline__ void dma_load_seg(Dma& d, const Seg& S, const TileCtx& t) {
  d.S = S;
  d.rA = make_rsrc(S.a + t.m0 * S.lda_b, t.m_rows * S.lda_b);
  const uint32_t rowA = static_cast<uint32_t>(64 * t.wave + (t.lane >> 3)) * S.lda_b;
#pragma unroll
  for (int i = 0; i < 8; ++i) d.offA[i] = rowA + static_cast<uint32_t>(8 * i) * S.lda_b + ((t.c0 ^ i) << 4);
  if (!NN) {
    const int64_t nb = EPI == EPI_SWIGLU_FWD ? t.j0 : t.n0;
    d.rB0 = make_rsrc(S.b0 + nb * S.ldb_b, t.n_rows * S.ldb_b);
    d.rB1 = EPI == EPI_SWIGLU_FWD ? make_rsrc(S.b1 + nb * S.ldb_b, t.n_rows * S.ldb_b) : d.rB0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = EPI == EPI_SWIGLU_FWD ? (2 * t.wave + i / 4) * 16 + 8 * (i & 1) + (t.lane >> 3)
                                            : 64 * t.wave + 8 * i + (t.lane >> 3);
      d.offB[i] = static_cast<uint32_t>(row) * S.ldb_b + ((t.c0 ^ i) << 4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 2 * (8 * t.wave + i) + (t.lane >> 5);
      const int nc = (t.lane & 31) ^ nn_swz(k);
      d.offB[i] = (t.n0 + nc * 8 < t.N) ? static_cast<uint32_t>(k) * S.ldb_b + nc * 16 : OOB;
    }
  }
}

// DMA instructions [i0, i0+4) of operand A (op 0) or B (op 1) of tile d.kt
// into stage `buf`. A K-major chunk is fetched iff its first element is below
// the tile's valid K; past the last tile the valid K is 0, so those loads
// only write zeros into the idle stage.
template <bool NN, int EPI>
__device__ __forceinline__ void dma_issue(const Dma& d, int op, int i0, char* buf, int nk, const TileCtx& t) {
  const int kv = d.kt < nk ? d.S.K - d.k0 : 0;
  const int soff = d.k0 * 2;
  if (op == 0) {
#pragma unroll
    for (int i = i0; i < i0 + 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rA, (lds_void_t*)(buf + (64 * t.wave + 8 * i) * 128), 16,
                                               ((t.c0 ^ i) << 3) < kv ? d.offA[i] : OOB, soff, 0, 0);
  } else if (!NN) {
    char* bbuf = buf + TILE_BYTES;
#pragma unroll
    for (int i = i0; i < i0 + 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds((EPI == EPI_SWIGLU_FWD && (i & 2)) ? d.rB1 : d.rB0,
                                               (lds_void_t*)(bbuf + (64 * t.wave + 8 * i) * 128), 16,
                                               ((t.c0 ^ i) << 3) < kv ? d.offB[i] : OOB, soff, 0, 0);
  } else {
    // clamp on the scalar unit: the descriptor must stay uniform
    const uint32_t krows = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(kv >= BK ? BK : (kv > 0 ? kv : 0)));
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(d.S.b0 + static_cast<int64_t>(d.k0) * d.S.ldb_b + t.n0 * 2, krows * d.S.ldb_b);
    char* bbuf = buf + TILE_BYTES;
#pragma unroll
    for (int i = i0; i < i0 + 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(bbuf + (8 * t.wave + i) * 1024), 16, d.offB[i], 0,
                                               0, 0);
  }
}

template <bool NN, int EPI>
__device__ __forceinline__ void dma_advance(Dma& d, int nseg, const Seg& s0, const Seg& s1, const Seg& s2,
                                            const TileCtx& t) {
  ++d.kt;
  d.k0 += BK;
  if (d.k0 >= d.S.K && d.seg + 1 < nseg) {
    d.k0 = 0;
    ++d.seg;
    dma_load_seg<NN, EPI>(d, seg_pick(d.seg, s0, s1, s2), t);
  }
}

// Lane-constant parts of the fragment read addresses.
// K-major tile, fragment row r = w*128 + a*16 + (lane & 15), chunk
// ks*4 + (lane >> 4): swz = (lane >> 4) ^ (lane & 7) ^ ((lane >> 3) & 1) ^
// 4*ks ^ (2a & 7), so the byte address is a per-lane base, XOR a constant of
// (ks, a mod 4), plus the immediate a*2048.
// N-major tile: k = ks*32 + hh*4 + (lane >> 4)*8 + (lrow >> 2),
// n = wn*128 + b*16 + 4*(lrow & 3): nn_swz(k) depends on the lane only and the
// chunk is wn*16 + ((2b) ^ nn_swz) + ((lrow & 3) >> 1).
struct ReadCtx {
  uint32_t rdA, rdB, rdN;
  int nsw;
};

__device__ __forceinline__ uint4 read_a(const ReadCtx& rc, const char* buf, int ks, int a) {
  return *reinterpret_cast<const uint4*>(buf + (rc.rdA ^ ((4 * ks ^ (2 * a & 7)) << 4)) + a * 2048);
}

template <bool NN>
__device__ __forceinline__ uint4 read_b(const ReadCtx& rc, const char* buf, int ks, int b) {
  const char* bbuf = buf + TILE_BYTES;
  if (!NN) return *reinterpret_cast<const uint4*>(bbuf + (rc.rdB ^ ((4 * ks ^ (2 * b & 7)) << 4)) + b * 2048);
  const uint32_t base = rc.rdN + ((((2 * b) ^ rc.nsw) & 15) << 4) + ks * 32 * 512;
  const v4i16_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(bbuf + base));
  const v4i16_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(bbuf + base + 4 * 512));
  const uint2 u0 = __builtin_bit_cast(uint2, t0);
  const uint2 u1 = __builtin_bit_cast(uint2, t1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

__device__ __forceinline__ void mfma_group(f32x4_t (&acc)[8][8], int a, const uint4 (&fa)[8], const uint4 (&fb)[8]) {
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[a][b] = mma<bf16_t>::step(fb[b], fa[a], acc[a][b]);
}

template <bool NN, int EPI>
__device__ __forceinline__ void gemm_bf16_body(const GemmParams& p) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

  TileCtx t;
  t.lane = threadIdx.x & 63;
  t.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.c0 = (t.lane & 7) ^ (t.lane >> 3);
  const int wm = t.wave >> 1;
  const int wn = t.wave & 1;

  // ---- tile selection: XCD-aware (block b runs on XCD b % 8), grouped along M
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int per = nblk / 8, rem = nblk % 8, x = bid % 8;
  const int logical = x * per + (x < rem ? x : rem) + bid / 8;
  const int gm = p.group_m;
  const int width = gm * p.tiles_n;
  const int group = logical / width;
  const int first_m = group * gm;
  const int gsize = min(p.tiles_m - first_m, gm);
  const int tm = first_m + (logical % width) % gsize;
  const int tn = (logical % width) / gsize;
  t.m0 = static_cast<int64_t>(tm) * BM;
  t.n0 = static_cast<int64_t>(tn) * BN;  // gate/up: twice the first column j0
  t.j0 = t.n0 >> 1;
  t.N = p.N;
  t.m_rows = static_cast<uint32_t>(min<int64_t>(BM, p.M - t.m0));
  t.n_rows = static_cast<uint32_t>(EPI == EPI_SWIGLU_FWD ? min<int64_t>(BN / 2, p.N - t.j0)
                                                         : min<int64_t>(BN, p.N - t.n0));

  const Seg s0 = seg_at(p, 0), s1 = seg_at(p, 1), s2 = seg_at(p, 2);
  const int nk = (s0.K + BK - 1) / BK + (s1.K + BK - 1) / BK + (s2.K + BK - 1) / BK;

  f32x4_t acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = t.lane & 15;
  const int lgrp = t.lane >> 4;
  ReadCtx rc;
  rc.rdA = static_cast<uint32_t>((wm * 128 + lrow) * 128 + ((lgrp ^ (lrow & 7) ^ (lrow >> 3)) << 4));
  rc.rdB = static_cast<uint32_t>((wn * 128 + lrow) * 128 + ((lgrp ^ (lrow & 7) ^ (lrow >> 3)) << 4));
  rc.nsw = 2 * ((lrow >> 2) | ((lgrp & 1) << 2));
  rc.rdN = static_cast<uint32_t>((lgrp * 8 + (lrow >> 2)) * 512 + (wn * 16 + ((lrow & 3) >> 1)) * 16 +
                                 8 * (lrow & 1));

  // ---- software pipeline. Tile t lives in stage t & 1; k-step 0 of a tile
  // (k 0..31) uses B fragments fb0, k-step 1 (k 32..63) uses fb1, and the A
  // fragments stream through fa: slot a is refilled for the next k-step as
  // soon as MFMA group a (8 MFMAs, all B fragments times A fragment a) has
  // been issued. Per tile kt:
  //   step 0: after group a, read A fragment a of step 1 and, for a < 4,
  //           B fragments 2a, 2a+1 of step 1
  //   step 1: after group 2, wait for this wave's DMA of tile kt+1 and
  //           barrier (tile kt+1 is in LDS everywhere and every read of tile
  //           kt has retired); groups 3-7 then carry the reads of tile kt+1's
  //           step-0 fragments and the DMA of tile kt+2 into tile kt's stage
  Dma d;
  d.seg = 0;
  d.k0 = 0;
  d.kt = 0;
  dma_load_seg<NN, EPI>(d, s0, t);
  uint4 fa[8], fb0[8], fb1[8];
  if (nk > 0) {
    dma_issue<NN, EPI>(d, 0, 0, smem, nk, t);
    dma_issue<NN, EPI>(d, 0, 4, smem, nk, t);
    dma_issue<NN, EPI>(d, 1, 0, smem, nk, t);
    dma_issue<NN, EPI>(d, 1, 4, smem, nk, t);
    dma_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    char* st1 = smem + STAGE_BYTES;
    dma_issue<NN, EPI>(d, 0, 0, st1, nk, t);
    dma_issue<NN, EPI>(d, 0, 4, st1, nk, t);
    dma_issue<NN, EPI>(d, 1, 0, st1, nk, t);
    dma_issue<NN, EPI>(d, 1, 4, st1, nk, t);
    dma_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t);
#pragma unroll
    for (int b = 0; b < 8; ++b) fb0[b] = read_b<NN>(rc, smem, 0, b);
#pragma unroll
    for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, smem, 0, a);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE_BYTES;
    const char* nxt = smem + ((kt + 1) & 1) * STAGE_BYTES;
    char* dma_buf = smem + (kt & 1) * STAGE_BYTES;  // tile kt+2 reuses tile kt's stage
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      mfma_group(acc, g, fa, fb0);
      LMLP_SCHED_FENCE();
      fa[g] = read_a(rc, cur, 1, g);
      if (g < 4) {
        fb1[2 * g] = read_b<NN>(rc, cur, 1, 2 * g);
        fb1[2 * g + 1] = read_b<NN>(rc, cur, 1, 2 * g + 1);
      }
      LMLP_SCHED_FENCE();
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      mfma_group(acc, g, fa, fb1);
      LMLP_SCHED_FENCE();
      if (g == 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): DMA of tile kt+1 landed
        __syncthreads();
      }
      if (g == 3) {
#pragma unroll
        for (int b = 0; b < 4; ++b) fb0[b] = read_b<NN>(rc, nxt, 0, b);
        fa[0] = read_a(rc, nxt, 0, 0);
        fa[1] = read_a(rc, nxt, 0, 1);
      }
      if (g == 4) {
#pragma unroll
        for (int b = 4; b < 8; ++b) fb0[b] = read_b<NN>(rc, nxt, 0, b);
        fa[2] = read_a(rc, nxt, 0, 2);
        fa[3] = read_a(rc, nxt, 0, 3);
        fa[4] = read_a(rc, nxt, 0, 4);
      }
      if (g == 5) {
        dma_issue<NN, EPI>(d, 0, 0, dma_buf, nk, t);
        dma_issue<NN, EPI>(d, 0, 4, dma_buf, nk, t);
        fa[5] = read_a(rc, nxt, 0, 5);
      }
      if (g == 6) {
        dma_issue<NN, EPI>(d, 1, 0, dma_buf, nk, t);
        dma_issue<NN, EPI>(d, 1, 4, dma_buf, nk, t);
        dma_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t);
        fa[6] = read_a(rc, nxt, 0, 6);
      }
      if (g == 7) fa[7] = read_a(rc, nxt, 0, 7);
      LMLP_SCHED_FENCE();
    }
  }

  // the last trip prefetched empty tiles: let that DMA retire before the
  // workgroup can exit and hand its LDS to another workgroup
  __builtin_amdgcn_s_waitcnt(0x0F70);

  gemm_epilogue<bf16_t, EPI>(p, acc, t.m0, t.n0, wm, wn, t.lane);
}

template <bool NN, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmParams p) {
  gemm_bf16_body<NN, EPI>(p);
}

}  // namespace

template <bool NN, int EPI>
static hipError_t launch_t(GemmParams p, hipStream_t stream) {
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  p.tiles_n = EPI == EPI_SWIGLU_FWD ? static_cast<int>((p.N + BN / 2 - 1) / (BN / 2))
                                    : static_cast<int>((p.N + BN - 1) / BN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
  const int nblk = p.tiles_m * p.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<NN, EPI>), dim3(nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmParams& p, int nn, int epi, hipStream_t stream) {
  if (!nn && epi == EPI_STORE) return launch_t<false, EPI_STORE>(p, stream);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch_t<false, EPI_SWIGLU_FWD>(p, stream);
  if (nn && epi == EPI_STORE) return launch_t<true, EPI_STORE>(p, stream);
  if (nn && epi == EPI_SWIGLU_BWD) return launch_t<true, EPI_SWIGLU_BWD>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lmlp
