// bf16 MFMA GEMM for gfx950 with an LDS-DMA ring.
//
// Same products, K segments and epilogues as the general kernel in gemm.hip
// (base K loop plus the appended rank-r adapter K-steps of the fused LoRA MLP,
// "Unsloth 深度分析报告", section 创新之处), specialised for dense bf16.
//
// Workgroup tile 256x256, 4 waves in 2x2, each wave 128x128 = 8x8 MFMA
// 16x16x32 tiles (256 fp32 accumulators per lane). K advances 32 elements
// (64 bytes) per k-tile: one MFMA k-step, 64 MFMAs per wave in 8 groups of 8
// (group a = A fragment a times all eight B fragments).
//
// Operand staging:
//  * buffer_load ... lds moves 16 bytes per lane straight from global memory
//    into LDS (no staging registers). Each instruction fills 1 KB of LDS
//    linearly; the XOR swizzle is applied by choosing which global chunk a
//    lane fetches. Rows past M/N, columns past N and K tails read as zero
//    through the buffer range check (invalid chunks get an offset past the
//    range), so nothing branches.
//  * K-major tiles (A always, B in the NT products) sit in LDS as
//    [256 rows][64 bytes]; chunk c of row r is stored at position
//    c ^ ((r >> 1) & 3). A ds_read_b128 is served eight lanes at a time, and
//    eight consecutive rows of one chunk then cover all 32 banks once (with
//    (r >> 2) the even and the odd rows collided pairwise: every operand read
//    took twice its time, counted as half of all LDS cycles).
//  * N-major B tiles (the NN products dZ = dY W_d and dX = dG W_g + dU W_u)
//    sit in LDS as in memory, [32 k][256 n], and are transposed on the way to
//    registers by ds_read_b64_tr_b16: in each 16-lane group, lane j names 4
//    consecutive n of row k0 + j/4 and lane i receives column i of the four
//    rows, i.e. 4 consecutive k of one n (the MFMA operand layout).
//  * A ring of STAGES k-tiles (32 KB each). The DMA of tile kt+STAGES-1 is
//    issued while tile kt is multiplied, one instruction per MFMA group, so
//    STAGES-2 tiles of loads are in flight besides the one being consumed.
//  * The DMA instruction comes from lds_dma.h (an asm block the compiler does
//    not track); completion is waited for explicitly: vmcnt before the
//    barrier that opens a k-tile, and vmcnt(0) before the epilogue.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "stage_ring.h"

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

namespace lmlp {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;                   // bf16 elements of K per k-tile (64 bytes)
constexpr int NTHREADS = 256;
constexpr int TILE_BYTES = BM * BK * 2;  // one operand tile: 16 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int STAGES = 5;                // 160 KB of LDS
constexpr uint32_t OOB = DMA_OOB;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4i16_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

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
  int64_t m0, n0, j0;  // j0: first gate/up column (n0 / 2)
  uint32_t m_rows, n_rows;
  int64_t N;
  int wave, lane, c1;  // c1 = (lane & 3) ^ ((lane >> 3) & 3)
};

// DMA state of the next k-tile to fetch
struct Dma {
  rsrc_t rA, rB0, rB1;
  uint32_t offA[4], offB[4];
  Seg S;
  int seg, k0, kt;
};

// Per-lane offsets of the DMA pattern for segment S.
// K-major tiles: instruction i of this wave fills tile rows
// 64*wave + 16*i + (lane >> 2), chunk position lane & 3; that position holds
// logical chunk (lane & 3) ^ ((row >> 1) & 3) = c1 for every i.
// Gate/up B operand: tile rows alternate gate/up every 16, so instruction i
// reads weight row (2*wave + i/2)*16 + lane/4 of the gate (i even) or up panel.
// N-major B tiles: instruction i fills rows k = 2*(4*wave + i) + (lane >> 5),
// chunk position lane & 31 holding n-chunk (lane & 31) ^ nn_swz(k); chunks
// past N are never fetched.
template <bool NN, int EPI>
__device__ __forceinline__ void dma_load_seg(Dma& d, const Seg& S, const TileCtx& t) {
  d.S = S;
  d.rA = make_rsrc(S.a + t.m0 * S.lda_b, t.m_rows * S.lda_b);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d.offA[i] = static_cast<uint32_t>(64 * t.wave + 16 * i + (t.lane >> 2)) * S.lda_b + (t.c1 << 4);
  if (!NN) {
    const int64_t nb = EPI == EPI_SWIGLU_FWD ? t.j0 : t.n0;
    d.rB0 = make_rsrc(S.b0 + nb * S.ldb_b, t.n_rows * S.ldb_b);
    d.rB1 = EPI == EPI_SWIGLU_FWD ? make_rsrc(S.b1 + nb * S.ldb_b, t.n_rows * S.ldb_b) : d.rB0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = EPI == EPI_SWIGLU_FWD ? (2 * t.wave + i / 2) * 16 + (t.lane >> 2)
                                            : 64 * t.wave + 16 * i + (t.lane >> 2);
      d.offB[i] = static_cast<uint32_t>(row) * S.ldb_b + (t.c1 << 4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 2 * (4 * t.wave + i) + (t.lane >> 5);
      const int nc = (t.lane & 31) ^ nn_swz(k);
      d.offB[i] = (t.n0 + nc * 8 < t.N) ? static_cast<uint32_t>(k) * S.ldb_b + nc * 16 : OOB;
    }
  }
}

// DMA instruction j (0..7) of k-tile d.kt into stage `buf`: j < 4 are A's,
// j >= 4 are B's. A K-major chunk is fetched iff its first element is below
// the tile's valid K; past the last tile the valid K is 0 and the loads only
// write zeros into an idle stage.
template <bool NN, int EPI>
__device__ __forceinline__ void dma_issue(const Dma& d, int j, char* buf, int nk, const TileCtx& t) {
  const int kv = d.kt < nk ? d.S.K - d.k0 : 0;
  const int soff = d.k0 * 2;
  const bool cval = (t.c1 << 3) < kv;
  if (j < 4) {
    const int i = j;
    dma16(d.rA, buf + (64 * t.wave + 16 * i) * 64, cval ? d.offA[i] : OOB, soff);
  } else if (!NN) {
    const int i = j - 4;
    dma16((EPI == EPI_SWIGLU_FWD && (i & 1)) ? d.rB1 : d.rB0, buf + TILE_BYTES + (64 * t.wave + 16 * i) * 64,
          cval ? d.offB[i] : OOB, soff);
  } else {
    const int i = j - 4;
    // clamp on the scalar unit: the descriptor must stay uniform
    const uint32_t krows =
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(kv >= BK ? BK : (kv > 0 ? kv : 0)));
    const rsrc_t r =
        make_rsrc(d.S.b0 + static_cast<int64_t>(d.k0) * d.S.ldb_b + t.n0 * 2, krows * d.S.ldb_b);
    dma16(r, buf + TILE_BYTES + (4 * t.wave + i) * 1024, d.offB[i], 0);
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
// K-major tile, fragment row r = w*128 + a*16 + (lane & 15), chunk lane >> 4:
// position (lane >> 4) ^ ((r >> 1) & 3) = (lane >> 4) ^ ((lane >> 1) & 3), so
// the address is a per-lane base plus the immediate a*1024.
// N-major tile: k = hh*4 + (lane >> 4)*8 + (lrow >> 2), n = wn*128 + b*16 +
// 4*(lrow & 3): nn_swz(k) depends on the lane only and the chunk is
// wn*16 + ((2b) ^ nn_swz) + ((lrow & 3) >> 1).
struct ReadCtx {
  uint32_t rdA, rdB, rdN;
  int nsw;
  int wc;  // N-major reads of 128-wide tiles: the wave's first column chunk (wn * 8)
};

__device__ __forceinline__ uint4 read_a(const ReadCtx& rc, const char* buf, int a) {
  return *reinterpret_cast<const uint4*>(buf + rc.rdA + a * 1024);
}

template <bool NN, int NB = 8>
__device__ __forceinline__ uint4 read_b(const ReadCtx& rc, const char* buf, int b) {
  const char* bbuf = buf + TILE_BYTES;
  if (!NN) return *reinterpret_cast<const uint4*>(bbuf + rc.rdB + b * 1024);
  // 256-wide tiles: the wave's first chunk (wn * 16) is a multiple of 16 and
  // sits in rdN; 128-wide ones (wn * 8): the swizzle has to see it
  const uint32_t base = NB == 8 ? rc.rdN + ((((2 * b) ^ rc.nsw) & 15) << 4)
                                : rc.rdN + (((rc.wc + 2 * b) ^ rc.nsw) << 4);
  const v4i16_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(bbuf + base));
  const v4i16_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(bbuf + base + 4 * 512));
  const uint2 u0 = __builtin_bit_cast(uint2, t0);
  const uint2 u1 = __builtin_bit_cast(uint2, t1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

// MFMA source chunk of a [k rows][n] bf16 tile read transposed: lane l
// passes the address of its 4 columns (4 * (l & 3) onward, relative to the
// lane's 16-column block) in k-row (l >> 4) * 8 + (l & 15) / 4 and receives 8
// consecutive k of column l & 15 (two ds_read_b64_tr_b16, the second `kstep4`
// bytes = 4 rows further).
__device__ __forceinline__ uint4 read_tr16x2(const char* p, int kstep4) {
  const v4i16_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
  const v4i16_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p + kstep4));
  const uint2 u0 = __builtin_bit_cast(uint2, t0);
  const uint2 u1 = __builtin_bit_cast(uint2, t1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

template <int NB>
__device__ __forceinline__ void mfma_group(f32x4_t (&acc)[8][NB], int a, const uint4 (&fa)[8], const uint4 (&fb)[8]) {
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[a][b] = mma<bf16_t>::step(fb[b], fa[a], acc[a][b]);
}


// One k-tile of the pipeline. Tile kt lives in stage st_cur. While it is
// multiplied (8 MFMA groups), the fragments of tile kt+1 are read (A slot g
// refilled after group g; the B fragments go to the other set fbn) and the
// DMA of tile kt+STAGES-1 is issued into tile kt-1's stage, one instruction
// per group. After group 0 each wave waits for its DMA of tile kt+1 and the
// workgroup meets at a barrier: tile kt+1 is then in LDS for every wave and
// every read of tile kt-1 has retired.
template <bool NN, int EPI, int NB>
__device__ __forceinline__ void pipeline_tile(f32x4_t (&acc)[8][NB], uint4 (&fa)[8], const uint4 (&fb)[8],
                                              uint4 (&fbn)[8], Dma& d, int& st_cur, char* smem,
                                              const ReadCtx& rc, const TileCtx& t, int nk, int nseg,
                                              const Seg& s0, const Seg& s1, const Seg& s2) {
  const int st_nxt = st_cur + 1 == STAGES ? 0 : st_cur + 1;
  const int st_dma = st_cur == 0 ? STAGES - 1 : st_cur - 1;  // tile kt-1's stage
  const char* nxt = smem + st_nxt * STAGE_BYTES;
  char* dbuf = smem + st_dma * STAGE_BYTES;
  mfma_group<NB>(acc, 0, fa, fb);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<8 * (STAGES - 3)>();  // DMA of tile kt+1 landed (this wave)
  __syncthreads();
#pragma unroll
  for (int g = 1; g < 8; ++g) {
    mfma_group<NB>(acc, g, fa, fb);
    __builtin_amdgcn_sched_barrier(0);
    dma_issue<NN, EPI>(d, g - 1, dbuf, nk, t);
    fa[g - 1] = read_a(rc, nxt, g - 1);
    if (2 * g <= NB) {
      fbn[2 * g - 2] = read_b<NN, NB>(rc, nxt, 2 * g - 2);
      fbn[2 * g - 1] = read_b<NN, NB>(rc, nxt, 2 * g - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  dma_issue<NN, EPI>(d, 7, dbuf, nk, t);
  dma_advance<NN, EPI>(d, nseg, s0, s1, s2, t);
  fa[7] = read_a(rc, nxt, 7);
  __builtin_amdgcn_sched_barrier(0);
  st_cur = st_nxt;
}

// ---- epilogue through LDS ----------------------------------------------
// Once the K loop has drained, the LDS ring is free. Accumulators go to LDS in
// their MFMA layout (lane l: row l & 15, columns 4*(l >> 4) .. +3 of each
// 16x16 tile) and come back row-contiguous, so every global access is 16
// bytes per lane and a wave instruction covers whole row segments (512 bytes
// of a 256-column output, 256 bytes of a 128-column gate/up output). Row
// pitches carry 16 bytes of padding to spread the tile-layout writes over the
// LDS banks. The SwiGLU arithmetic is the one of the register epilogue: G and
// U rounded to bf16 first, Z = SiLU(G) U from the rounded values; backward
// dG = dZ U sig (1 + G (1 - sig)), dU = dZ SiLU(G).
constexpr int EP_PITCH_C = 256 * 2 + 16;   // bf16 [256 rows][256]
constexpr int EP_PITCH_GU = 128 * 2 + 16;  // bf16 [256 rows][128], G and U side by side
constexpr int EP_PITCH_DZ = 256 * 4 + 16;  // fp32 [128 rows][256], one half of dZ at a time
constexpr int EP_SP = 256 * 2 + 16;        // bf16 [32 rows][256]: dG, dU or Z of one backward pass
constexpr int EP_SBUF = 3 * 32 * EP_SP;     // dG, dU and Z of one pass
constexpr int EP_PF = 2;                    // backward passes whose G and U are in flight
// LDS the staging needs: a kernel's shared array must be at least this large
constexpr int EP_LDS_BYTES = 256 * EP_PITCH_C > 2 * 256 * EP_PITCH_GU
                                 ? (256 * EP_PITCH_C > 128 * EP_PITCH_DZ ? 256 * EP_PITCH_C : 128 * EP_PITCH_DZ)
                                 : (2 * 256 * EP_PITCH_GU > 128 * EP_PITCH_DZ ? 2 * 256 * EP_PITCH_GU
                                                                             : 128 * EP_PITCH_DZ);
static_assert(STAGES * STAGE_BYTES >= EP_LDS_BYTES, "the dense ring must hold the epilogue staging");
static_assert(STAGES * STAGE_BYTES >= 2 * EP_SBUF + 80 * 512, "two pass buffers plus the rank rows");

__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 f32x8_to_bf16(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// [rows][cols] bf16 in LDS (pitch bytes) -> global, 16 bytes per lane,
// CHUNKS 16-byte chunks per row, NT threads. Rows past m_rows and chunks past
// the valid columns are not stored.
template <int CHUNKS, int NTH = NTHREADS>
__device__ __forceinline__ void lds_rows_to_global(const char* lds, int pitch, int rows, bf16_t* dst,
                                                   int64_t ldc, uint32_t m_rows, int64_t ncols) {
  const int tid = threadIdx.x;
  const int chunk = tid % CHUNKS;
  const int rsub = tid / CHUNKS;
  constexpr int RSTEP = NTH / CHUNKS;
  const bool cval = chunk * 8 < ncols;
#pragma unroll 4
  for (int r = rsub; r < rows; r += RSTEP) {
    const uint4 v = *reinterpret_cast<const uint4*>(lds + r * pitch + chunk * 16);
    if (cval && static_cast<uint32_t>(r) < m_rows)
      *reinterpret_cast<uint4*>(dst + r * ldc + chunk * 8) = v;
  }
}

// Workgroup barrier that orders LDS accesses only: global loads and stores
// issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Epilogue operands that do not depend on the product, fetched before the K
// loop so that their latency is hidden: the rank rows of the fused backward,
// 16-byte chunk c of row n (thread tid + 256 j) for the LDS position
// c ^ (n & 7); what lies past N (columns) or M (tokens) is zero. Rows 0-31:
// B_g^T, B_u^T over the tile's columns; rows 32-79: P_g^T, P_u^T, Q_d^T over
// the tile's tokens.
// 1024 chunks of B^T rows and 1536 of P^T / Q_d^T rows over NTH threads
template <int NTH = NTHREADS>
struct EpiPre {
  static constexpr int NBT = 1024 / NTH;
  static constexpr int NPT = 1536 / NTH;
  uint4 rk[NBT + NPT];
};

template <int EPI, int QRB, int NTH = NTHREADS>
__device__ __forceinline__ void epi_preload(const GemmParams& p, const TileCtx& t, EpiPre<NTH>& pre) {
  if (EPI != EPI_SWIGLU_BWD || QRB != 1) return;
  constexpr int NBT = EpiPre<NTH>::NBT, NPT = EpiPre<NTH>::NPT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < NBT + NPT; ++j) {
    const int idx = tid + NTH * (j < NBT ? j : j - NBT);
    const int row = idx >> 5, c = idx & 31;
    const bf16_t* src;
    bool ok;
    if (j < NBT) {
      src = static_cast<const bf16_t*>(row < 16 ? p.pj_b0 : p.pj_b1) + (row & 15) * p.pj_ldb + t.n0 + 8 * c;
      ok = static_cast<uint32_t>(8 * c) < t.n_rows;
    } else {
      src = row < 32 ? static_cast<const bf16_t*>(p.pj_pguT) + row * p.pj_ldt + t.m0 + 8 * c
                     : static_cast<const bf16_t*>(p.pj_qdT) + (row - 32) * p.pj_ldt + t.m0 + 8 * c;
      ok = static_cast<uint32_t>(8 * c) < t.m_rows;
    }
    pre.rk[j] = ok ? *reinterpret_cast<const uint4*>(src) : zero4();
  }
}

// NB: 16-column blocks per wave; NTH: threads of the workgroup. Four waves
// (NTH 256) hold 2 x 2 blocks of 128 x 16 NB: NB 8 for 256-wide tiles, NB 4
// for 128-wide ones (the plain and backward epilogues only, with the upper
// half of the staging left idle). Eight waves (NTH 512) hold 2 x 4 blocks of
// 128 x 64 (NB 4) of a 256-wide tile.
template <int EPI, int QRB = 0, int NB = 8, int NTH = NTHREADS>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, f32x4_t (&acc)[8][NB], const TileCtx& t,
                                             int wm, int wn, char* smem, const EpiPre<NTH>& pre) {
  static_assert(NB == 8 || NTH == 512 || EPI != EPI_SWIGLU_FWD, "gate/up tiles are 256 wide");
  const int lrow = t.lane & 15;
  const int lcol = 4 * (t.lane >> 4);
  if (EPI == EPI_STORE_F32) {
    // a split-K partial, the accumulators unrounded: staged through LDS one
    // 128-row half at a time (as the backward stages dZ), then stored
    // row-contiguous, 16 bytes (four columns) per lane
    float* C = static_cast<float*>(p.c0) + t.m0 * p.ldc + t.n0;
    constexpr int CH = 8 * NB;  // 16-byte chunks of a staged row
    __syncthreads();            // every wave is done with the ring
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wm == h) {
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            *reinterpret_cast<f32x4_t*>(smem + (a * 16 + lrow) * EP_PITCH_DZ + (wn * 16 * NB + b * 16 + lcol) * 4) =
                acc[a][b];
      }
      __syncthreads();
      for (int i = threadIdx.x; i < 128 * CH; i += NTH) {
        const int rl = i / CH, c = i % CH;
        const int r = h * 128 + rl;
        if (static_cast<uint32_t>(r) < t.m_rows && static_cast<uint32_t>(4 * c) < t.n_rows)
          *reinterpret_cast<float4*>(C + r * p.ldc + 4 * c) =
              *reinterpret_cast<const float4*>(smem + rl * EP_PITCH_DZ + c * 16);
      }
      __syncthreads();
    }
  } else if (EPI == EPI_STORE) {
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int r = wm * 128 + a * 16 + lrow;
        const int c = wn * 16 * NB + b * 16 + lcol;
        *reinterpret_cast<uint2*>(smem + r * EP_PITCH_C + c * 2) =
            make_uint2(pack_bf16x2(acc[a][b][0], acc[a][b][1]), pack_bf16x2(acc[a][b][2], acc[a][b][3]));
      }
    __syncthreads();
    bf16_t* C = static_cast<bf16_t*>(p.c0) + t.m0 * p.ldc + t.n0;
    lds_rows_to_global<32, NTH>(smem, EP_PITCH_C, 256, C, p.ldc, t.m_rows, t.n_rows);
  } else if (EPI == EPI_SWIGLU_FWD) {
    // tiles (a, 2q) hold G and (a, 2q+1) hold U of gate/up columns
    // j0 + wn*8*NB + 16q + lcol .. +3; both go to LDS rounded to bf16, then
    // one pass per row chunk stores G and U and forms Z = SiLU(G) U from the
    // same rounded values
    char* gbuf = smem;
    char* ubuf = smem + 256 * EP_PITCH_GU;
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int q = 0; q < NB / 2; ++q) {
        const int off = (wm * 128 + a * 16 + lrow) * EP_PITCH_GU + (wn * 8 * NB + q * 16 + lcol) * 2;
        const f32x4_t& g = acc[a][2 * q];
        const f32x4_t& u = acc[a][2 * q + 1];
        *reinterpret_cast<uint2*>(gbuf + off) = make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
        *reinterpret_cast<uint2*>(ubuf + off) = make_uint2(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]));
      }
    __syncthreads();
    const int tid = threadIdx.x;
    const int chunk = tid & 15;  // 8 columns of a 128-column row
    const int rsub = tid >> 4;
    const bool cval = static_cast<uint32_t>(chunk * 8) < t.n_rows;
    // outputs are optional (uniform branches): the backward's recompute of G
    // and U has no Z, the forward of the recompute mode no G, U
    bf16_t* Gp = p.c0 ? static_cast<bf16_t*>(p.c0) + t.m0 * p.ldc + t.j0 + chunk * 8 : nullptr;
    bf16_t* Up = p.c1 ? static_cast<bf16_t*>(p.c1) + t.m0 * p.ldc + t.j0 + chunk * 8 : nullptr;
    bf16_t* Zp = p.c2 ? static_cast<bf16_t*>(p.c2) + t.m0 * p.ldc + t.j0 + chunk * 8 : nullptr;
#pragma unroll 4
    for (int r = rsub; r < 256; r += NTH / 16) {
      const uint4 gv = *reinterpret_cast<const uint4*>(gbuf + r * EP_PITCH_GU + chunk * 16);
      const uint4 uv = *reinterpret_cast<const uint4*>(ubuf + r * EP_PITCH_GU + chunk * 16);
      if (cval && static_cast<uint32_t>(r) < t.m_rows) {
        const int64_t off = r * p.ldc;
        if (Gp) *reinterpret_cast<uint4*>(Gp + off) = gv;
        if (Up) *reinterpret_cast<uint4*>(Up + off) = uv;
        if (Zp) {
          float g[8], u[8], z[8];
          bf16x8_to_f32(gv, g);
          bf16x8_to_f32(uv, u);
#pragma unroll
          for (int e = 0; e < 8; ++e) z[e] = g[e] * sigmoidf_fast(g[e]) * u[e];
          *reinterpret_cast<uint4*>(Zp + off) =
              make_uint4(pack_bf16x2_pk(z[0], z[1]), pack_bf16x2_pk(z[2], z[3]), pack_bf16x2_pk(z[4], z[5]),
                         pack_bf16x2_pk(z[6], z[7]));
        }
      }
    }
  } else if (QRB == 0) {  // EPI_SWIGLU_BWD: acc = dZ; reload G, U; recompute the gate
    const bf16_t* Gp = static_cast<const bf16_t*>(p.g_in) + t.m0 * p.ldc + t.n0;
    const bf16_t* Up = static_cast<const bf16_t*>(p.u_in) + t.m0 * p.ldc + t.n0;
    bf16_t* dGp = static_cast<bf16_t*>(p.c0) + t.m0 * p.ldc + t.n0;
    bf16_t* dUp = static_cast<bf16_t*>(p.c1) + t.m0 * p.ldc + t.n0;
    bf16_t* Zp = p.c2 ? static_cast<bf16_t*>(p.c2) + t.m0 * p.ldc + t.n0 : nullptr;
    // thread -> 8 consecutive columns (chunk) of rows rsub, rsub + RS, ... of a half
    constexpr int RS = NTH / 32;   // rows per step
    constexpr int RPT = 128 / RS;  // rows per thread in a half
    const int tid = threadIdx.x;
    const int chunk = tid & 31;
    const int rsub = tid >> 5;
    const bool cval = static_cast<uint32_t>(chunk * 8) < t.n_rows;
    // G and U of one half-tile (RPT rows per thread), fetched before they are
    // needed; invalid positions read element 0 and are never stored
    uint4 gv[RPT], uv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = RS * i + rsub;
      const int64_t off = (cval && static_cast<uint32_t>(r) < t.m_rows) ? r * p.ldc + chunk * 8 : 0;
      gv[i] = *reinterpret_cast<const uint4*>(Gp + off);
      uv[i] = *reinterpret_cast<const uint4*>(Up + off);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wm == h) {
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            *reinterpret_cast<f32x4_t*>(smem + (a * 16 + lrow) * EP_PITCH_DZ + (wn * 16 * NB + b * 16 + lcol) * 4) =
                acc[a][b];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int rl = RS * i + rsub;  // row within the half
        const int r = h * 128 + rl;   // row within the tile
        const float4 d0 = *reinterpret_cast<const float4*>(smem + rl * EP_PITCH_DZ + chunk * 32);
        const float4 d1 = *reinterpret_cast<const float4*>(smem + rl * EP_PITCH_DZ + chunk * 32 + 16);
        const float dz[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        float g[8], u[8], dg[8], du[8], z[8];
        bf16x8_to_f32(gv[i], g);
        bf16x8_to_f32(uv[i], u);
        if (h == 0) {  // this slot is free: fetch the same position of the second half
          const int r2 = 128 + rl;
          const int64_t off = (cval && static_cast<uint32_t>(r2) < t.m_rows) ? r2 * p.ldc + chunk * 8 : 0;
          gv[i] = *reinterpret_cast<const uint4*>(Gp + off);
          uv[i] = *reinterpret_cast<const uint4*>(Up + off);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = sigmoidf_fast(g[e]);
          const float act = g[e] * sg;
          dg[e] = dz[e] * u[e] * sg * (1.0f + g[e] * (1.0f - sg));
          du[e] = dz[e] * act;
          z[e] = act * u[e];
        }
        if (cval && static_cast<uint32_t>(r) < t.m_rows) {
          const int64_t off = r * p.ldc + chunk * 8;
          *reinterpret_cast<uint4*>(dGp + off) = f32x8_to_bf16(dg);
          *reinterpret_cast<uint4*>(dUp + off) = f32x8_to_bf16(du);
          if (Zp) *reinterpret_cast<uint4*>(Zp + off) = f32x8_to_bf16(z);
        }
      }
      if (h == 0) __syncthreads();  // the second half overwrites the staging area
    }
  } else {  // EPI_SWIGLU_BWD with the rank-16 products of dG, dU and Z (see above)
    // Eight passes; pass a takes accumulator row block a of every wave, i.e.
    // tile rows 16a .. 16a+15 (wm = 0) and 128 + 16a .. +15 (wm = 1): 32
    // staging rows, staging row s = tile row (s >> 4) * 128 + 16a + (s & 15).
    // G and U come from global memory straight into registers in the
    // accumulator layout (lane l: row l & 15, columns 4 (l >> 4) .. +3 of each
    // 16-column block, 8 bytes per block), EP_PF passes ahead, so the gate
    // arithmetic runs on registers and dZ never goes through LDS. dG, dU and Z
    // (bf16) go to one of two LDS buffers per pass, from which the rank
    // products read their operands and the row-contiguous stores of dG and dU
    // are made.
    constexpr int NW = NTH / 64;     // waves: 2 along M, NW / 2 along N
    constexpr int TW = NB * NW / 2;  // 16-column blocks of the tile
    constexpr int JB = TW / NW;      // 16-column blocks of column products per wave
    constexpr int NBT = EpiPre<NTH>::NBT, NPT = EpiPre<NTH>::NPT;
    const bf16_t* Gp = static_cast<const bf16_t*>(p.g_in) + t.m0 * p.ldc + t.n0;
    const bf16_t* Up = static_cast<const bf16_t*>(p.u_in) + t.m0 * p.ldc + t.n0;
    bf16_t* dGp = static_cast<bf16_t*>(p.c0) + t.m0 * p.ldc + t.n0;
    bf16_t* dUp = static_cast<bf16_t*>(p.c1) + t.m0 * p.ldc + t.n0;
    char* bt = smem + 2 * EP_SBUF;  // B_g^T, B_u^T rows [32][512 B] over the tile's columns
    char* pt = bt + 32 * 512;       // P_g^T, P_u^T, Q_d^T rows [48][512 B] over the tile's tokens
    const int tid = threadIdx.x;
    const int lch = t.lane >> 4;
    // G and U of pass a into (g, u), by buffer loads over the tile's rows: 16
    // bytes per lane, lane l reading row l & 15 at columns 8 (l >> 4) .. +7 of
    // each 32-column pair of accumulator blocks (an instruction covers 16 rows
    // x 64 bytes; 8-byte loads in the accumulator layout itself, 16 rows x 32
    // bytes, fetch at half the rate per compute unit). Two permlane16 and two
    // permlane32 swaps then give every lane its accumulator-layout columns
    // 4 (l >> 4) .. +3 of both blocks. The whole offset is in the lane's VGPR,
    // which the range check covers: rows past M fall past num_records and read
    // zero, and chunks past N (a multiple of 8) get an offset past it.
    const int crow = wm * 128 + lrow;         // tile row of the lane in pass 0
    const int ccol = wn * 16 * NB + 8 * lch;  // first column of the lane's chunk in pair 0
    const int nrec = static_cast<int>(t.m_rows * p.ldc * 2);
    const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Gp), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rU = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Up), 0, nrec, 0x00020000);
    const int vb = (crow * static_cast<int>(p.ldc) + ccol) * 2;
    // dwords d0..d3 of the lanes' chunks -> accumulator-layout pairs of blocks
    // 2j (x) and 2j + 1 (y): with D_g the chunk of lane group g (= l >> 4),
    // group g needs D_{g>>1} dwords 2(g&1), +1 for block 2j and D_{2+(g>>1)}
    // for block 2j + 1
    auto to_acc_layout = [](const uint4& d, uint2& x, uint2& y) {
      const auto s0 = __builtin_amdgcn_permlane16_swap(d.x, d.z, false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(d.y, d.w, false, false);
      const auto t0 = __builtin_amdgcn_permlane32_swap(s0[0], s0[1], false, false);
      const auto t1 = __builtin_amdgcn_permlane32_swap(s1[0], s1[1], false, false);
      x = make_uint2(t0[0], t1[0]);
      y = make_uint2(t0[1], t1[1]);
    };
    // chunk j (0 .. NB/2 - 1) of G (up false) or U of pass a
    auto load_one = [&](int a, int j, bool up) {
      const bool ok = static_cast<uint32_t>(ccol + 32 * j) < t.n_rows;
      const int vo = ok ? vb + (16 * a * static_cast<int>(p.ldc) + 32 * j) * 2 : static_cast<int>(OOB);
      return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(up ? rU : rG, vo, 0, 0));
    };
    auto fetch = [&](int a, uint4 (&g)[NB / 2], uint4 (&u)[NB / 2]) {
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        g[j] = load_one(a, j, false);
        u[j] = load_one(a, j, true);
      }
    };
    // (the last of the first EP_PF passes after the rank rows are written: the
    // compiler's wait for those, at most 63 newer loads, then waits for none)
    uint4 pg[EP_PF][NB / 2], pu[EP_PF][NB / 2];
    static_assert(NB * (EP_PF - 1) <= 63, "vmcnt range");
#pragma unroll
    for (int a = 0; a < EP_PF - 1; ++a) fetch(a, pg[a], pu[a]);
    lds_barrier();  // every wave is done with the ring
#pragma unroll
    for (int j = 0; j < NBT + NPT; ++j) {
      const int idx = tid + NTH * (j < NBT ? j : j - NBT);
      const int row = idx >> 5, c = idx & 31;
      char* dst = (j < NBT ? bt : pt) + row * 512 + ((c ^ (row & 7)) << 4);
      *reinterpret_cast<uint4*>(dst) = pre.rk[j];
    }
    fetch(EP_PF - 1, pg[EP_PF - 1], pu[EP_PF - 1]);
    // column products, summed over the tile's tokens: wave w owns the
    // 16-column blocks JB w .. JB w + JB - 1
    f32x4_t cg[JB], cu[JB], cz[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) cg[j] = cu[j] = cz[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // store k (0 .. NB-1) of pass a's dG (k even) or dU (k odd), row-contiguous
    // from the staging: staging row tid / CH + RS (k >> 1), 16-byte chunk tid % CH
    constexpr int CH = 2 * TW;    // 16-byte chunks of a staging row
    constexpr int RS = NTH / CH;  // staging rows per step
    static_assert(2 * (32 / RS) == NB, "one store per accumulator block");
    const int chunk = tid % CH;
    const bool cv = static_cast<uint32_t>(chunk * 8) < t.n_rows;
    auto store_one = [&](int a, int k) {
      const char* src = smem + (a & 1) * EP_SBUF + (k & 1) * 32 * EP_SP;
      const int sr = tid / CH + RS * (k >> 1);
      const int r = (sr >> 4) * 128 + 16 * a + (sr & 15);
      const uint4 v = *reinterpret_cast<const uint4*>(src + sr * EP_SP + chunk * 16);
      if (cv && static_cast<uint32_t>(r) < t.m_rows)
        *reinterpret_cast<uint4*>(((k & 1) ? dUp : dGp) + r * p.ldc + chunk * 8) = v;
    };
    const int srow = wm * 16 + lrow;  // staging row of the lane's accumulator rows
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      __builtin_amdgcn_sched_barrier(0);
      char* sgb = smem + (a & 1) * EP_SBUF;  // dG [32][EP_SP]
      char* sub = sgb + 32 * EP_SP;          // dU
      char* szb = sub + 32 * EP_SP;          // Z
      uint2 gl[NB], ul[NB];
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        to_acc_layout(pg[a % EP_PF][j], gl[2 * j], gl[2 * j + 1]);
        to_acc_layout(pu[a % EP_PF][j], ul[2 * j], ul[2 * j + 1]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint2 gq = gl[b], uq = ul[b];
        const float g[4] = {__uint_as_float(gq.x << 16), __uint_as_float(gq.x & 0xFFFF0000u),
                            __uint_as_float(gq.y << 16), __uint_as_float(gq.y & 0xFFFF0000u)};
        const float u[4] = {__uint_as_float(uq.x << 16), __uint_as_float(uq.x & 0xFFFF0000u),
                            __uint_as_float(uq.y << 16), __uint_as_float(uq.y & 0xFFFF0000u)};
        float dg[4], du[4], z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dz = acc[a][b][e];
          const float sg = sigmoidf_fast(g[e]);
          const float act = g[e] * sg;
          dg[e] = dz * u[e] * sg * (1.0f + g[e] * (1.0f - sg));
          du[e] = dz * act;
          z[e] = act * u[e];
        }
        const int off = srow * EP_SP + (wn * 16 * NB + 16 * b + 4 * lch) * 2;
        *reinterpret_cast<uint2*>(sgb + off) = make_uint2(pack_bf16x2_pk(dg[0], dg[1]), pack_bf16x2_pk(dg[2], dg[3]));
        *reinterpret_cast<uint2*>(sub + off) = make_uint2(pack_bf16x2_pk(du[0], du[1]), pack_bf16x2_pk(du[2], du[3]));
        *reinterpret_cast<uint2*>(szb + off) = make_uint2(pack_bf16x2_pk(z[0], z[1]), pack_bf16x2_pk(z[2], z[3]));
        // one load of pass a + EP_PF (into the registers this pass has just
        // converted) and one store of pass a - 1 per block: spread through
        // the arithmetic, the vector memory instructions find the queue
        // drained instead of stalling in a burst behind each other
        if (a + EP_PF < 8) {
          if (b & 1) pu[a % EP_PF][b >> 1] = load_one(a + EP_PF, b >> 1, true);
          else pg[a % EP_PF][b >> 1] = load_one(a + EP_PF, b >> 1, false);
        }
        if (a > 0) store_one(a - 1, b);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();  // the pass's staging (and, at pass 0, the rank rows) complete
      __builtin_amdgcn_sched_barrier(0);
      // Row products: Q_g[token][n] = sum over the tile's columns of dG * B_g
      // (B_g^T row n = l & 15), likewise Q_u: wave w < 4 takes token block
      // w & 1 of the pass and product w >> 1; the staged chunk (row l & 15,
      // chunk 4 ks + l / 16) is the MFMA source as it stands.
      if (t.wave < 4) {
        const int tb = t.wave & 1;
        const int pr = t.wave >> 1;
        const char* src = (pr ? sub : sgb) + (tb * 16 + lrow) * EP_SP;
        const char* brow = bt + (pr * 16 + lrow) * 512;
        f32x4_t q = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < TW / 2; ++ks) {
          const int ch = ks * 4 + lch;
          const uint4 bv = *reinterpret_cast<const uint4*>(brow + ((ch ^ (lrow & 7)) << 4));
          q = mma<bf16_t>::step(bv, *reinterpret_cast<const uint4*>(src + ch * 16), q);
        }
        // lane l holds Q[token = staging row 16 tb + (l & 15)][n = 4 (l >> 4) .. +3]:
        // one split-K slice (this tile column)
        const int r = tb * 128 + 16 * a + lrow;
        if (static_cast<uint32_t>(r) < t.m_rows) {
          const int64_t base = ((p.pj_slice0 + t.n0 / (16 * TW)) * p.pj_T + t.m0 + r) * 16 + 4 * lch;
          *reinterpret_cast<f32x4_t*>((pr ? p.pj_part1 : p.pj_part0) + base) = q;
        }
      }
      // Column products over the pass's 32 tokens (one k-step):
      // dB_g^T[n][col] += sum over tokens of P_g^T[n][t] dG[t][col], likewise
      // dB_u^T with dU and dA_d[n][col] with Q_d^T and Z. Lane l supplies k
      // slots 8 (l >> 4) .. +7 = staging rows, i.e. tokens tok0 .. tok0 + 7;
      // the column operand is read transposed (ds_read_b64_tr_b16): column
      // 16 ib + (l & 15) of those staging rows.
      {
        const int tok0 = (lch >> 1) * 128 + 16 * a + 8 * (lch & 1);
        const int ppos = (((tok0 >> 3) ^ (lrow & 7)) << 4);
        const uint4 pgv = *reinterpret_cast<const uint4*>(pt + lrow * 512 + ppos);
        const uint4 puv = *reinterpret_cast<const uint4*>(pt + (16 + lrow) * 512 + ppos);
        const uint4 pqv = *reinterpret_cast<const uint4*>(pt + (32 + lrow) * 512 + ppos);
        const int krow = lch * 8 + (lrow >> 2);  // staging row of the first transposed read
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          const int c0 = (JB * t.wave + j) * 16 + 4 * (lrow & 3);  // first of this lane's 4 columns
          const int o = krow * EP_SP + c0 * 2;
          cg[j] = mma<bf16_t>::step(pgv, read_tr16x2(sgb + o, 4 * EP_SP), cg[j]);
          cu[j] = mma<bf16_t>::step(puv, read_tr16x2(sub + o, 4 * EP_SP), cu[j]);
          cz[j] = mma<bf16_t>::step(pqv, read_tr16x2(szb + o, 4 * EP_SP), cz[j]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) store_one(7, k);
    // lane l holds [n = 4 (l >> 4) .. +3][col = 16 ib + (l & 15)] summed over
    // the tile's tokens: one slice (this tile row) of each [col][16] partial
    const int64_t mt = t.m0 / BM;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int col = (JB * t.wave + j) * 16 + lrow;
      if (static_cast<uint32_t>(col) < t.n_rows) {
        const int64_t off = (mt * p.pj_ncol + t.n0 + col) * 16 + 4 * lch;
        *reinterpret_cast<f32x4_t*>(p.pj_cdg + off) = cg[j];
        *reinterpret_cast<f32x4_t*>(p.pj_cdu + off) = cu[j];
        *reinterpret_cast<f32x4_t*>(p.pj_cz + off) = cz[j];
      }
    }
  }
}

// Output tile of this workgroup: XCD-aware (block b runs on XCD b % 8), each
// XCD sweeping bands of group_m tiles along M so that its L2 reuses B panels.
template <int EPI, int NB = 8>
__device__ __forceinline__ void select_tile(const GemmParams& p, TileCtx& t, int bid, int nblk) {
  constexpr int TN = 32 * NB;  // tile width (gate/up: interleaved gate and up columns)
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
  t.n0 = static_cast<int64_t>(tn) * TN;  // gate/up: twice the first column j0
  t.j0 = t.n0 >> 1;
  t.N = EPI == EPI_SWIGLU_FWD ? p.N : min<int64_t>(p.N, t.n0 + TN);  // end of this tile's columns
  t.m_rows = static_cast<uint32_t>(min<int64_t>(BM, p.M - t.m0));
  t.n_rows = static_cast<uint32_t>(EPI == EPI_SWIGLU_FWD ? min<int64_t>(TN / 2, p.N - t.j0)
                                                         : min<int64_t>(TN, p.N - t.n0));

}

// One output tile: workgroup `bid` of `nblk` that share the tile sequence of p
// (bid % 8 must be the XCD the workgroup runs on for the XCD-aware order).
template <bool NN, int EPI, int QRB, int NB>
__device__ __forceinline__ void gemm_bf16_body(const GemmParams& p, int bid, int nblk, char* smem) {
  TileCtx t;
  t.lane = threadIdx.x & 63;
  t.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.c1 = (t.lane & 3) ^ ((t.lane >> 3) & 3);
  const int wm = t.wave >> 1;
  const int wn = t.wave & 1;

  select_tile<EPI, NB>(p, t, bid, nblk);
  EpiPre<> pre;
  epi_preload<EPI, QRB>(p, t, pre);

  const Seg s0 = seg_at(p, 0), s1 = seg_at(p, 1), s2 = seg_at(p, 2);
  int nk = (s0.K + BK - 1) / BK + (s1.K + BK - 1) / BK + (s2.K + BK - 1) / BK;
  nk += nk & 1;  // the loop runs k-tiles in pairs; an odd count gets one empty tile

  f32x4_t acc[8][NB];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = t.lane & 15;
  const int lgrp = t.lane >> 4;
  ReadCtx rc;
  rc.rdA = static_cast<uint32_t>((wm * 128 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.rdB = static_cast<uint32_t>((wn * 16 * NB + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.nsw = 2 * ((lrow >> 2) | ((lgrp & 1) << 2));
  rc.wc = wn * 2 * NB;
  rc.rdN = static_cast<uint32_t>((lgrp * 8 + (lrow >> 2)) * 512 + ((NB == 8 ? wn * 16 : 0) + ((lrow & 3) >> 1)) * 16 +
                                 8 * (lrow & 1));

  // ---- prologue: DMA of tiles 0 .. STAGES-2, then tile 0's fragments
  Dma d;
  d.seg = 0;
  d.kt = 0;
  d.k0 = 0;
  dma_load_seg<NN, EPI>(d, s0, t);
  uint4 fa[8], fbA[8], fbB[8];
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) dma_issue<NN, EPI>(d, j, smem + s * STAGE_BYTES, nk, t);
    dma_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t);
  }
  wait_vmcnt<8 * (STAGES - 2)>();  // tile 0 landed (this wave)
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) fbA[b] = read_b<NN, NB>(rc, smem, b);
#pragma unroll
  for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, smem, a);

  int st_cur = 0;
  for (int kt = 0; kt < nk; kt += 2) {
    pipeline_tile<NN, EPI, NB>(acc, fa, fbA, fbB, d, st_cur, smem, rc, t, nk, p.nseg, s0, s1, s2);
    pipeline_tile<NN, EPI, NB>(acc, fa, fbB, fbA, d, st_cur, smem, rc, t, nk, p.nseg, s0, s1, s2);
  }

  // the last tiles prefetched empty k-tiles: let that DMA retire before the
  // workgroup can exit and hand its LDS to another workgroup
  wait_vmcnt<0>();

  epilogue_lds<EPI, QRB, NB>(p, acc, t, wm, wn, smem, pre);
}

template <bool NN, int EPI, int QRB, int NB>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  gemm_bf16_body<NN, EPI, QRB, NB>(p, blockIdx.x, gridDim.x, smem);
}

// Several independent products of one kind in one launch (the experts of a
// grouped MLP): group g owns workgroups start[g] .. start[g+1]-1, of which the
// first tiles(g) compute its tiles in its own XCD-aware order; start[g] is a
// multiple of 8 so that a workgroup's position in its group keeps the XCD it
// runs on, and the padding workgroups exit at once.
template <bool NN, int EPI, int QRB, int NB>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_grouped_kernel(GemmGroups gg) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  const int bid = blockIdx.x;
  int g = 0;
  while (g + 1 < gg.n && bid >= gg.start[g + 1]) ++g;
  const GemmParams& p = gg.p[g];
  const int local = bid - gg.start[g];
  const int tiles = p.tiles_m * p.tiles_n;
  if (local >= tiles) return;
  gemm_bf16_body<NN, EPI, QRB, NB>(p, local, tiles, smem);
}

// ---- eight waves, two per SIMD, in ping-pong ---------------------------------
// The same 256x256 output tile, k-tiles, LDS layout and DMA ring as above,
// with eight waves of 128 x 64 (acc[8][4], 128 fp32 accumulators per lane, so
// two waves fit one SIMD's registers). Waves 0-3 (group 0) and 4-7 (group 1)
// have one wave on each SIMD. Every k-tile c is a memory phase followed by a
// compute phase for each wave:
//   memory(c):  read this wave's fragments of tile c (8 A, 4 B chunks) from
//               LDS and issue its 4 DMA instructions of a later tile
//   compute(c): the 32 MFMAs of tile c on those fragments
// with a workgroup barrier after each phase. Group 1 passes one extra
// barrier at the start, so at every barrier-delimited phase one group
// multiplies while the other reads and issues: each SIMD has one wave
// issuing MFMAs back to back and one wave issuing memory instructions.
// The fragment reads of memory(c) are waited for at the start of compute(c),
// after the barrier, so the memory phase only issues them.
// Ring (tile c in stage c % 5): group 0 reads tile c in phase 2c, group 1 in
// 2c+1, and both have consumed it by the barrier ending 2c+2. Group 0
// fetches the A tile (wave q: rows 64q .. 64q+63) of tile c+3 in memory(c),
// phase 2c, into the stage tile c-2 left; group 1 fetches the B tile
// (K-major rows 64q .. 64q+63; N-major k rows 8q .. 8q+7) of tile c+4 in
// memory(c), phase 2c+1, into the stage tile c-1 left. Tile c+1 is first
// read in phase 2c+2, so each wave waits for its share of it as late as it
// can: group 1 at the end of memory(c), group 0 at the end of compute(c)
// (phase 2c+1), both before that phase's barrier. Four 1 KB instructions per
// wave per k-tile, as the four-wave kernel's instructions j = 0-3 (A) and
// 4-7 (B) of wave q.
constexpr int NT8 = 512;
constexpr int STAGES8 = 5;
static_assert(STAGES8 * STAGE_BYTES <= STAGES * STAGE_BYTES, "ring of the eight-wave kernel");

template <bool NN, int EPI>
__device__ __forceinline__ void dma8_load_seg(Dma& d, const Seg& S, const TileCtx& t, int grp, int q) {
  TileCtx tq = t;
  tq.wave = q;
  dma_load_seg<NN, EPI>(d, S, tq);
  (void)grp;
}

// this wave's four DMA instructions of the next k-tile (a uniform branch on
// the group, so every offset index is a constant)
template <bool NN, int EPI>
__device__ __forceinline__ void dma8_issue4(const Dma& d, char* buf, int nk, const TileCtx& t, int grp, int q) {
  TileCtx tq = t;
  tq.wave = q;
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_issue<NN, EPI>(d, i, buf, nk, tq);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_issue<NN, EPI>(d, 4 + i, buf, nk, tq);
  }
}

template <bool NN, int EPI>
__device__ __forceinline__ void dma8_advance(Dma& d, int nseg, const Seg& s0, const Seg& s1, const Seg& s2,
                                             const TileCtx& t, int grp, int q) {
  ++d.kt;
  d.k0 += BK;
  if (d.k0 >= d.S.K && d.seg + 1 < nseg) {
    d.k0 = 0;
    ++d.seg;
    dma8_load_seg<NN, EPI>(d, seg_pick(d.seg, s0, s1, s2), t, grp, q);
  }
}

template <bool NN, int EPI, int QRB>
__device__ __forceinline__ void gemm8_body(const GemmParams& p, int bid, int nblk, char* smem) {
  TileCtx t;
  t.lane = threadIdx.x & 63;
  t.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.c1 = (t.lane & 3) ^ ((t.lane >> 3) & 3);
  const int grp = t.wave >> 2;  // ping-pong group, and the operand it fetches
  const int q = t.wave & 3;
  const int wm = grp;           // output rows 128 wm .. +127
  const int wn = q;             // output columns 64 wn .. +63
  select_tile<EPI, 8>(p, t, bid, nblk);
  EpiPre<NT8> pre;
  epi_preload<EPI, QRB, NT8>(p, t, pre);

  const Seg s0 = seg_at(p, 0), s1 = seg_at(p, 1), s2 = seg_at(p, 2);
  const int nk = (s0.K + BK - 1) / BK + (s1.K + BK - 1) / BK + (s2.K + BK - 1) / BK;

  f32x4_t acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = t.lane & 15;
  const int lgrp = t.lane >> 4;
  ReadCtx rc;
  rc.rdA = static_cast<uint32_t>((wm * 128 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.rdB = static_cast<uint32_t>((wn * 64 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.nsw = 2 * ((lrow >> 2) | ((lgrp & 1) << 2));
  rc.wc = wn * 8;
  rc.rdN = static_cast<uint32_t>((lgrp * 8 + (lrow >> 2)) * 512 + ((lrow & 3) >> 1) * 16 + 8 * (lrow & 1));

  // ---- prologue: group 0 issues tiles 0-2, group 1 tiles 0-3; tile 0 landed
  Dma d;
  d.seg = 0;
  d.kt = 0;
  d.k0 = 0;
  dma8_load_seg<NN, EPI>(d, s0, t, grp, q);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    dma8_issue4<NN, EPI>(d, smem + s * STAGE_BYTES, nk, t, grp, q);
    dma8_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t, grp, q);
  }
  if (grp == 1) {
    dma8_issue4<NN, EPI>(d, smem + 3 * STAGE_BYTES, nk, t, grp, q);
    dma8_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t, grp, q);
    wait_vmcnt<12>();
  } else {
    wait_vmcnt<8>();
  }
  __syncthreads();
  if (grp == 1) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  int st = 0;                   // stage of tile c
  int st_dma = 3 + grp;         // stage of the tile this wave fetches next (c + 3 + grp)
  for (int c = 0; c < nk; ++c) {
    const char* buf = smem + st * STAGE_BYTES;
    uint4 fa[8], fb[4];
#pragma unroll
    for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, buf, a);
#pragma unroll
    for (int b = 0; b < 4; ++b) fb[b] = read_b<NN, 4>(rc, buf, b);
    dma8_issue4<NN, EPI>(d, smem + st_dma * STAGE_BYTES, nk, t, grp, q);
    dma8_advance<NN, EPI>(d, p.nseg, s0, s1, s2, t, grp, q);
    if (grp == 1) wait_vmcnt<12>();  // group 1's share of tile c + 1 landed
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mma<bf16_t>::step(fb[b], fa[a], acc[a][b]);
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) wait_vmcnt<8>();  // group 0's share of tile c + 1 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    st = st + 1 == STAGES8 ? 0 : st + 1;
    st_dma = st_dma + 1 == STAGES8 ? 0 : st_dma + 1;
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();
  // the DMA past the last tile wrote zeros into idle stages: let it retire
  // before the ring is reused
  wait_vmcnt<0>();

  epilogue_lds<EPI, QRB, 4, NT8>(p, acc, t, wm, wn, smem, pre);
}

template <bool NN, int EPI, int QRB>
__global__ __launch_bounds__(NT8, 1) void gemm8_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  gemm8_body<NN, EPI, QRB>(p, blockIdx.x, gridDim.x, smem);
}

// grouped forms (the experts of a grouped MLP) of the eight-wave kernel, as
// gemm_bf16_grouped_kernel and gemm_bf16_table_kernel below
template <bool NN, int EPI, int QRB>
__global__ __launch_bounds__(NT8, 1) void gemm8_grouped_kernel(GemmGroups gg) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  const int bid = blockIdx.x;
  int g = 0;
  while (g + 1 < gg.n && bid >= gg.start[g + 1]) ++g;
  const GemmParams& p = gg.p[g];
  const int local = bid - gg.start[g];
  const int tiles = p.tiles_m * p.tiles_n;
  if (local >= tiles) return;
  gemm8_body<NN, EPI, QRB>(p, local, tiles, smem);
}

// decoded-tile row of packed row pr (gate/up: interleave the two panels)
template <int EPI>
__device__ __forceinline__ int q4_dense_row(int pr) {
  if (EPI != EPI_SWIGLU_FWD) return pr;
  const int panel = pr >> 7, r = pr & 127;
  return (r >> 4) * 32 + panel * 16 + (r & 15);
}

// ---- eight waves with a 4-bit B operand --------------------------------------
// The leading K segments hold 4-bit block weights (seg.bint4): codes and
// scales are staged through the ring, and each group decodes its half of a
// later k-tile in its compute phases into one of three bf16 B tiles outside
// the ring, laid out exactly as the DMA of a dense B tile would leave it
// (K-major rows for NT, N-major k rows for NN), so the fragment reads and the
// MFMA sequence are the dense kernel's and so are the results, bit for bit.
// Decoding is the block rule of the 4-bit format, w = bf16_rne(q * scale)
// with the product exact in fp32 (dq_chunk).
//  * ring stage (22 KB): the A tile (16 KB), the codes (4 KB: NT [256 B rows:
//    gate rows, then up rows][16 B]; NN [32 k rows][128 B]) and two 1 KB
//    scale slots (fp32; NT: slot h = B rows 128h .. 128h+127; NN: slot h =
//    k rows 16h .. 16h+15, four 64-column blocks each)
//  * three DMA instructions per wave and k-tile: group 0 fetches rows
//    64q .. 64q+47 of the A tile of tile c+3 in memory(c); group 1 rows
//    64q+48 .. 64q+63 of the A tile, its quarter of the codes and the scales
//    (waves 4-5; waves 6-7 issue an instruction whose lanes all fail the
//    range check into a dummy 1 KB) of tile c+4
//  * the decode runs in the compute phases, between the MFMAs (one MFMA,
//    two decode instructions; decoding in the memory phases instead, beside
//    the other group's MFMAs, measured 5 % slower per product): group 0
//    decodes its half of tile c+1 in compute(c) (phase 2c+1), group 1 its
//    half of tile c+2 in compute(c) (phase 2c+2), each into buffer
//    tile % 3; tile c+1 is first read in phase 2c+2, after both halves. The
//    codes are in LDS in time because group 1 waited for its share of tile
//    c+2 at the end of memory(c) (phase 2c+1); buffer (c+1) % 3 last held
//    tile c-2, consumed by the barrier ending phase 2c-2, buffer (c+2) % 3
//    tile c-1, consumed by the one ending 2c; every decode write has
//    completed before its phase's barrier
//  * the dense segments after the 4-bit ones (the adapter K steps) run after
//    the loop, one k-tile at a time through stage 0
constexpr int Q8_CODES = TILE_BYTES;               // codes in a stage
constexpr int Q8_SC = TILE_BYTES + 4096;           // two scale slots
constexpr int Q8_STAGE = TILE_BYTES + 6144;        // 22 KB
constexpr int Q8_DEC = STAGES8 * Q8_STAGE;         // three decoded B tiles
constexpr int Q8_DUMMY = Q8_DEC + 3 * TILE_BYTES;  // 1 KB target of the idle scale instructions
static_assert(Q8_DUMMY + 1024 <= STAGES * STAGE_BYTES, "LDS of the 4-bit eight-wave kernel");

// a descriptor known to be uniform, kept in scalar registers
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* base, uint32_t nbytes) {
  rsrc_t r = make_rsrc(base, nbytes);
  r.x = __builtin_amdgcn_readfirstlane(r.x);
  r.y = __builtin_amdgcn_readfirstlane(r.y);
  r.z = __builtin_amdgcn_readfirstlane(r.z);
  r.w = __builtin_amdgcn_readfirstlane(r.w);
  return r;
}

struct Q8Dma {
  rsrc_t rA;          // A panel of this tile row block
  uint32_t offA[3];
  uint32_t lda_b;
  rsrc_t rq;          // group 1: this wave's quarter of the codes
  uint32_t offq;
  uint32_t ldq_b;     // bytes per code row
  rsrc_t rs;          // group 1 waves 0-1: scales
  uint32_t offs;
  uint32_t ld_sc_b;   // bytes per scale row (NT: block row of N scales; NN: k row)
  int seg, k0, kt;
};

// descriptors of 4-bit segment S for this wave's role
template <bool NN, int EPI>
__device__ __forceinline__ void q8_load_seg(Q8Dma& d, const GemmSeg& g, const TileCtx& t, int grp, int q,
                                            int64_t Ntot) {
  // A rows: group 0 instructions i = 0-2 of wave q, group 1 instruction 3
  d.lda_b = static_cast<uint32_t>(g.lda * 2);
  d.rA = make_rsrc_u(static_cast<const char*>(g.a) + t.m0 * d.lda_b, t.m_rows * d.lda_b);
#pragma unroll
  for (int i = 0; i < 3; ++i)
    d.offA[i] = static_cast<uint32_t>(64 * q + 16 * (grp == 0 ? i : 3) + (t.lane >> 2)) * d.lda_b + (t.c1 << 4);
  if (grp == 0) {
    d.rq = d.rs = d.rA;  // unused by this group
    d.offq = d.offs = OOB;
    d.ldq_b = d.ld_sc_b = 0;
    return;
  }
  d.ldq_b = static_cast<uint32_t>(g.ldb / 2);
  if (!NN) {
    // code rows: B tile rows in codes order, 64 per wave
    const bool fwd = EPI == EPI_SWIGLU_FWD;
    const int64_t row0 = fwd ? t.j0 + 64 * (q & 1) : t.n0 + 64 * q;
    const int64_t nvalid = fwd ? static_cast<int64_t>(t.n_rows) - 64 * (q & 1)
                               : static_cast<int64_t>(t.n_rows) - 64 * q;
    const uint32_t rows = static_cast<uint32_t>(nvalid < 0 ? 0 : (nvalid > 64 ? 64 : nvalid));
    const char* cb = static_cast<const char*>(fwd && q >= 2 ? g.b1 : g.b0);
    d.rq = make_rsrc_u(cb + row0 * d.ldq_b, rows * d.ldq_b);
    d.offq = static_cast<uint32_t>(t.lane) * d.ldq_b;
    // scales, block-major fp32 [K/64][Ntot]: slot q (q < 2) = 128 B rows
    d.ld_sc_b = static_cast<uint32_t>(Ntot * 4);
    const int64_t srow0 = fwd ? t.j0 : t.n0 + 128 * q;
    const int64_t svalid = fwd ? static_cast<int64_t>(t.n_rows) : static_cast<int64_t>(t.n_rows) - 128 * q;
    const char* sb = static_cast<const char*>(fwd && q == 1 ? g.bs1 : g.bs0);
    d.rs = make_rsrc_u(sb + srow0 * 4, static_cast<uint32_t>(g.K / 64) * d.ld_sc_b);
    d.offs = (q < 2 && t.lane < 32 && 4 * t.lane < svalid) ? static_cast<uint32_t>(t.lane) * 16 : OOB;
  } else {
    // code rows: k rows 8q .. 8q+7, 128 bytes (256 columns) each
    d.rq = make_rsrc_u(static_cast<const char*>(g.b0) + t.n0 / 2, static_cast<uint32_t>(g.K) * d.ldq_b);
    const int cchunk = t.lane & 7;
    d.offq = (32 * cchunk < static_cast<int>(t.n_rows))
                 ? static_cast<uint32_t>(8 * q + (t.lane >> 3)) * d.ldq_b + cchunk * 16
                 : OOB;
    // scales, row-major fp32 [K][ld_sc], ld_sc a multiple of 4: slot q (q < 2)
    // = k rows 16q .. 16q+15, the tile's four 64-column blocks each
    const int64_t ld_sc = (Ntot / 64 + 3) / 4 * 4;
    d.ld_sc_b = static_cast<uint32_t>(ld_sc * 4);
    d.rs = make_rsrc_u(static_cast<const char*>(g.bs0) + (t.n0 / 64) * 4, static_cast<uint32_t>(g.K) * d.ld_sc_b);
    d.offs = (q < 2 && t.lane < 16) ? static_cast<uint32_t>(16 * q + t.lane) * d.ld_sc_b : OOB;
  }
}

// this wave's DMA of k-tile d.kt (past the 4-bit tiles: every lane fails the
// range check and the instructions only write zeros into idle stages)
template <bool NN>
__device__ __forceinline__ void q8_issue(const Q8Dma& d, char* st, char* dummy, int nkq, const TileCtx& t, int grp,
                                         int q) {
  const bool live = d.kt < nkq;
  const uint32_t soff = static_cast<uint32_t>(d.k0) * 2;
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16(d.rA, st + (64 * q + 16 * i) * 64, live ? d.offA[i] : OOB, soff);
  } else {
    dma16(d.rA, st + (64 * q + 48) * 64, live ? d.offA[0] : OOB, soff);
    const uint32_t soq = NN ? static_cast<uint32_t>(d.k0) * d.ldq_b : static_cast<uint32_t>(d.k0 / 2);
    dma16(d.rq, st + Q8_CODES + q * 1024, live ? d.offq : OOB, soq);
    const uint32_t sos = NN ? static_cast<uint32_t>(d.k0) * d.ld_sc_b : static_cast<uint32_t>(d.k0 / 64) * d.ld_sc_b;
    dma16(d.rs, q < 2 ? st + Q8_SC + q * 1024 : dummy, live ? d.offs : OOB, sos);
  }
}

// this thread's 16 codes and their scale of a staged k-tile (the half its
// group decodes)
struct Q8Codes {
  uint2 codes;
  float sc;
};
template <bool NN>
__device__ __forceinline__ Q8Codes q8_read_codes(const char* st, int grp, int tid_g) {
  Q8Codes c;
  if (NN) {
    const int kr = 16 * grp + (tid_g >> 4);  // k row
    const int cp = tid_g & 15;               // pair of 8-column chunks
    c.codes = *reinterpret_cast<const uint2*>(st + Q8_CODES + kr * 128 + cp * 8);
    c.sc = *reinterpret_cast<const float*>(st + Q8_SC + grp * 1024 + (kr & 15) * 16 + (cp >> 2) * 4);
  } else {
    const int cr = 128 * grp + (tid_g >> 1);  // code row
    const int h = tid_g & 1;                  // 16 k of the row's 32
    c.codes = *reinterpret_cast<const uint2*>(st + Q8_CODES + cr * 16 + h * 8);
    c.sc = *reinterpret_cast<const float*>(st + Q8_SC + grp * 1024 + (cr & 127) * 4);
  }
  return c;
}

// decode them into the dense B tile layout
template <bool NN, int EPI>
__device__ __forceinline__ void q8_decode(const Q8Codes& c, char* dec, int grp, int tid_g) {
  if (NN) {
    const int kr = 16 * grp + (tid_g >> 4);
    const int cp = tid_g & 15;
    const int sw = nn_swz(kr);
    *reinterpret_cast<uint4*>(dec + kr * 512 + (((2 * cp) ^ sw) << 4)) = dq_chunk(c.codes.x, c.sc);
    *reinterpret_cast<uint4*>(dec + kr * 512 + (((2 * cp + 1) ^ sw) << 4)) = dq_chunk(c.codes.y, c.sc);
  } else {
    const int cr = 128 * grp + (tid_g >> 1);
    const int h = tid_g & 1;
    const int drow = q4_dense_row<EPI>(cr);
    const int sw = (drow >> 1) & 3;
    *reinterpret_cast<uint4*>(dec + drow * 64 + (((2 * h) ^ sw) << 4)) = dq_chunk(c.codes.x, c.sc);
    *reinterpret_cast<uint4*>(dec + drow * 64 + (((2 * h + 1) ^ sw) << 4)) = dq_chunk(c.codes.y, c.sc);
  }
}

template <bool NN, int EPI, int QRB>
__device__ __forceinline__ void gemm8q4_body(const GemmParams& p, int bid, int nblk, char* smem) {
  TileCtx t;
  t.lane = threadIdx.x & 63;
  t.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.c1 = (t.lane & 3) ^ ((t.lane >> 3) & 3);
  const int grp = t.wave >> 2;
  const int q = t.wave & 3;
  const int wm = grp;
  const int wn = q;
  const int tid_g = threadIdx.x & 255;
  select_tile<EPI, 8>(p, t, bid, nblk);
  EpiPre<NT8> pre;
  epi_preload<EPI, QRB, NT8>(p, t, pre);

  // the 4-bit segments lead; nq (1 or 2) of them
  int nq = 0;
  while (nq < p.nseg && nq < 2 && p.seg[nq].bint4) ++nq;
  int nkq = 0;
  for (int s2 = 0; s2 < nq; ++s2) nkq += static_cast<int>(p.seg[s2].K / BK);  // multiples of 64

  f32x4_t acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = t.lane & 15;
  const int lgrp = t.lane >> 4;
  ReadCtx rc;
  rc.rdA = static_cast<uint32_t>((wm * 128 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.rdB = static_cast<uint32_t>((wn * 64 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.nsw = 2 * ((lrow >> 2) | ((lgrp & 1) << 2));
  rc.wc = wn * 8;
  rc.rdN = static_cast<uint32_t>((lgrp * 8 + (lrow >> 2)) * 512 + ((lrow & 3) >> 1) * 16 + 8 * (lrow & 1));

  char* dummy = smem + Q8_DUMMY;
  // the segments by constant index (held in registers: a runtime index
  // would load from the argument block, and the wait for that load would
  // drain the fragment reads in flight)
  const GemmSeg g0 = p.seg[0], g1 = p.seg[1];
  Q8Dma d;
  d.seg = 0;
  d.kt = 0;
  d.k0 = 0;
  int cur_k = static_cast<int>(g0.K);
  q8_load_seg<NN, EPI>(d, g0, t, grp, q, p.N);
  // at most two 4-bit segments (dG and dU of the dX product)
  auto advance = [&]() {
    ++d.kt;
    d.k0 += BK;
    if (d.k0 >= cur_k && d.seg + 1 < nq) {
      d.k0 = 0;
      ++d.seg;
      cur_k = static_cast<int>(g1.K);
      q8_load_seg<NN, EPI>(d, g1, t, grp, q, p.N);
    }
  };

  // ---- prologue: A of tiles 0-2, codes of tiles 0-3; tile 0 decoded
#pragma unroll
  for (int s2 = 0; s2 < 3; ++s2) {
    q8_issue<NN>(d, smem + s2 * Q8_STAGE, dummy, nkq, t, grp, q);
    advance();
  }
  if (grp == 1) {
    q8_issue<NN>(d, smem + 3 * Q8_STAGE, dummy, nkq, t, grp, q);
    advance();
  }
  wait_vmcnt<6>();  // group 0: tile 0; group 1: tiles 0 and 1
  __syncthreads();
  // tile 0 by both groups; group 1's half of tile 1, which group 1 would
  // have decoded in compute(-1)
  if (nkq > 0) q8_decode<NN, EPI>(q8_read_codes<NN>(smem, grp, tid_g), smem + Q8_DEC, grp, tid_g);
  if (grp == 1 && nkq > 1)
    q8_decode<NN, EPI>(q8_read_codes<NN>(smem + Q8_STAGE, grp, tid_g), smem + Q8_DEC + TILE_BYTES, grp, tid_g);
  __syncthreads();
  if (grp == 1) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  int st = 0;                // stage of tile c
  int st_dma = 3 + grp;      // stage of the tile this wave fetches next
  int dc = 0;                // decoded buffer of tile c
  for (int c = 0; c < nkq; ++c) {
    const char* buf = smem + st * Q8_STAGE;
    const char* dbuf = smem + Q8_DEC + dc * TILE_BYTES;
    const int st1 = st + 1 == STAGES8 ? 0 : st + 1;
    const int dc1 = dc + 1 == 3 ? 0 : dc + 1;
    uint4 fa[8], fb[4];
#pragma unroll
    for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, buf, a);
#pragma unroll
    for (int b = 0; b < 4; ++b) fb[b] = read_b<NN, 4>(rc, dbuf - TILE_BYTES, b);
    q8_issue<NN>(d, smem + st_dma * Q8_STAGE, dummy, nkq, t, grp, q);
    advance();
    if (grp == 1) wait_vmcnt<6>();  // tile c + 2 landed (group 1's share)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // compute(c): the MFMAs of tile c and this group's decode of tile td
    const int td = c + 1 + grp;
    const int st_td = grp == 0 ? st1 : (st1 + 1 == STAGES8 ? 0 : st1 + 1);
    const int dc_td = grp == 0 ? dc1 : (dc1 + 1 == 3 ? 0 : dc1 + 1);
    // (past the last tile the decode writes stale codes into a buffer no
    // one reads again: the dense tail and the epilogue use other LDS, after
    // this phase's writes have completed)
    (void)td;
    const Q8Codes cd = q8_read_codes<NN>(smem + st_td * Q8_STAGE, grp, tid_g);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mma<bf16_t>::step(fb[b], fa[a], acc[a][b]);
    q8_decode<NN, EPI>(cd, smem + Q8_DEC + dc_td * TILE_BYTES, grp, tid_g);
    // issue order: the code reads first, then one MFMA and two VALU
    // instructions (the decode) at a time, the decoded chunks' writes last
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 30; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the decode writes complete
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) wait_vmcnt<6>();  // group 0's share of tile c + 1 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    st = st1;
    st_dma = st_dma + 1 == STAGES8 ? 0 : st_dma + 1;
    dc = dc1;
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();
  wait_vmcnt<0>();
  __syncthreads();

  // ---- the dense segments after the 4-bit ones, one k-tile at a time
  for (int sg = nq; sg < p.nseg; ++sg) {
    const Seg S = seg_at(p, sg);
    Dma dd;
    dd.seg = sg;
    dd.kt = 0;
    dd.k0 = 0;
    dma8_load_seg<NN, EPI>(dd, S, t, grp, q);
    for (int k0 = 0; k0 < S.K; k0 += BK) {
      dd.k0 = k0;
      dma8_issue4<NN, EPI>(dd, smem, 1, t, grp, q);
      wait_vmcnt<0>();
      __syncthreads();
      uint4 fa[8], fb[4];
#pragma unroll
      for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, smem, a);
#pragma unroll
      for (int b = 0; b < 4; ++b) fb[b] = read_b<NN, 4>(rc, smem, b);
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mma<bf16_t>::step(fb[b], fa[a], acc[a][b]);
      __syncthreads();  // every wave is done with stage 0 before the next DMA
    }
  }

  epilogue_lds<EPI, QRB, 4, NT8>(p, acc, t, wm, wn, smem, pre);
}

template <bool NN, int EPI, int QRB>
__global__ __launch_bounds__(NT8, 1) void gemm8q4_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  gemm8q4_body<NN, EPI, QRB>(p, blockIdx.x, gridDim.x, smem);
}


// The matrix-core ceiling: each wave multiplies 8 A and 4 B operand chunks of
// random bits into 32 accumulators, rotating the A chunks every round so the
// inputs keep changing, with no memory traffic inside the loop.
__global__ __launch_bounds__(NT8, 1) void mfma_probe_kernel(const uint4* __restrict__ ops, float* sink, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint4* src = ops + (static_cast<int64_t>(blockIdx.x) * 8 + wave) * 768;
  uint4 a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = src[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = src[512 + i * 64 + lane];
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mma<bf16_t>::step(b[j], a[i], acc[i][j]);
    const uint4 t0 = a[0];
#pragma unroll
    for (int i = 0; i < 7; ++i) a[i] = a[i + 1];
    a[7] = make_uint4(t0.y, t0.z, t0.w, t0.x);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  sink[static_cast<int64_t>(blockIdx.x) * NT8 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(const void* ops, float* sink, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(NT8), 0, stream, static_cast<const uint4*>(ops), sink,
                     iters);
  return hipGetLastError();
}

template <bool NN, int EPI, int QRB = 0, int NB = 8>
static hipError_t launch_t(GemmParams p, hipStream_t stream) {
  constexpr int TN = 32 * NB;
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  p.tiles_n = EPI == EPI_SWIGLU_FWD ? static_cast<int>((p.N + TN / 2 - 1) / (TN / 2))
                                    : static_cast<int>((p.N + TN - 1) / TN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
  const int nblk = p.tiles_m * p.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<NN, EPI, QRB, NB>), dim3(nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

template <bool NN, int EPI, int QRB = 0>
static hipError_t launch8_t(GemmParams p, hipStream_t stream) {
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  p.tiles_n = EPI == EPI_SWIGLU_FWD ? static_cast<int>((p.N + BN / 2 - 1) / (BN / 2))
                                    : static_cast<int>((p.N + BN - 1) / BN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
  const int nblk = p.tiles_m * p.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm8_kernel<NN, EPI, QRB>), dim3(nblk), dim3(NT8), 0, stream, p);
  return hipGetLastError();
}

// Groups whose parameter blocks sit in device memory (more groups than the
// kernel arguments hold): the same workgroup -> (group, tile) map, with the
// group starts in the arguments.
//
// With many small groups (the experts of a fine-grained MoE), each group's
// tiles can instead all run on one XCD (`pinned`): workgroup b runs on XCD
// b % 8 as its slot b / 8 there; the groups of XCD x are xfirst[x] ..
// xfirst[x+1]-1 and group g takes slots start[g] .. of its XCD. A group's
// tiles then occupy consecutive slots of one XCD, so they run at about the
// same time and share its L2: the expert's weight panels are fetched once
// for all its row tiles, and each row panel once for all its column tiles,
// where spread over eight XCDs every XCD fetched its own copies.
struct GroupStarts {
  int32_t start[kMaxTableGroups + 1];
  int32_t n;
  int32_t pinned;
  int32_t xfirst[9];
};

// (group, tile within the group) of workgroup bid; false for an idle one
__device__ __forceinline__ bool group_of(const GroupStarts& gs, int bid, int& g, int& local) {
  int lo, hi, s;
  if (gs.pinned) {
    s = bid >> 3;
    lo = gs.xfirst[bid & 7];
    hi = gs.xfirst[(bid & 7) + 1] - 1;
    if (lo > hi) return false;
  } else {
    s = bid;
    lo = 0;
    hi = gs.n - 1;
  }
  while (lo < hi) {  // the last group whose start is <= s
    const int mid = (lo + hi + 1) >> 1;
    if (gs.start[mid] <= s) lo = mid;
    else hi = mid - 1;
  }
  g = lo;
  local = s - gs.start[lo];
  return true;
}

template <bool NN, int EPI, int QRB, int NB>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_table_kernel(const GemmParams* __restrict__ table,
                                                                     GroupStarts gs) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  int g, local;
  if (!group_of(gs, blockIdx.x, g, local)) return;
  const GemmParams& p = table[g];
  const int tiles = p.tiles_m * p.tiles_n;
  if (local >= tiles) return;
  // pinned: the group's tiles in plain order on one XCD (bid 8 * local of
  // 8 * tiles maps to tile `local`)
  if (gs.pinned) gemm_bf16_body<NN, EPI, QRB, NB>(p, 8 * local, 8 * tiles, smem);
  else gemm_bf16_body<NN, EPI, QRB, NB>(p, local, tiles, smem);
}

template <bool NN, int EPI, int QRB>
__global__ __launch_bounds__(NT8, 1) void gemm8_table_kernel(const GemmParams* __restrict__ table, GroupStarts gs) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  int g, local;
  if (!group_of(gs, blockIdx.x, g, local)) return;
  const GemmParams& p = table[g];
  const int tiles = p.tiles_m * p.tiles_n;
  if (local >= tiles) return;
  if (gs.pinned) gemm8_body<NN, EPI, QRB>(p, 8 * local, 8 * tiles, smem);
  else gemm8_body<NN, EPI, QRB>(p, local, tiles, smem);
}

// the gate/up and dZ products run on eight waves as in a single launch
template <int EPI, int NB>
constexpr bool kGrouped8 = NB == 8 && (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD);
// plain stores run on eight waves too when each group is pinned to one XCD
// (short K loops of small experts); spread, the four-wave kernel is faster
template <int EPI, int NB>
constexpr bool kPinned8 = NB == 8 && EPI == EPI_STORE;

template <bool NN, int EPI, int QRB, int NB>
static void launch_table_kernel(const GemmParams* tp, const GroupStarts& gs, int nblk, hipStream_t stream) {
  if constexpr (kGrouped8<EPI, NB> || kPinned8<EPI, NB>) {
    if (kGrouped8<EPI, NB> || gs.pinned) {
      hipLaunchKernelGGL((gemm8_table_kernel<NN, EPI, QRB>), dim3(nblk), dim3(NT8), 0, stream, tp, gs);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_bf16_table_kernel<NN, EPI, QRB, NB>), dim3(nblk), dim3(NTHREADS), 0, stream, tp, gs);
}

// copy of up to kMaxGemmGroups parameter blocks into a device table
struct TableChunk {
  GemmParams p[kMaxGemmGroups];
  GemmParams* dst;
  int32_t n;
};
__global__ __launch_bounds__(256) void write_table_kernel(TableChunk c) {
  constexpr int W = sizeof(GemmParams) / 4;
  static_assert(sizeof(GemmParams) % 4 == 0, "word copy");
  const uint32_t* src = reinterpret_cast<const uint32_t*>(c.p);
  uint32_t* dst = reinterpret_cast<uint32_t*>(c.dst);
  for (int i = threadIdx.x; i < c.n * W; i += blockDim.x) dst[i] = src[i];
}

// tile counts and band height of one product, as launch_t sets them
template <int EPI, int NB>
static void set_tiles(GemmParams& p) {
  constexpr int TN = 32 * NB;
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  p.tiles_n = EPI == EPI_SWIGLU_FWD ? static_cast<int>((p.N + TN / 2 - 1) / (TN / 2))
                                    : static_cast<int>((p.N + TN - 1) / TN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
}

template <bool NN, int EPI, int QRB = 0, int NB = 8>
static hipError_t launch_grouped_t(const GemmParams* ps, int n, hipStream_t stream) {
  // up to kMaxGemmGroups products with tiles per launch; each product is
  // taken once (products without tiles are skipped, not counted)
  for (int i = 0; i < n;) {
    GemmGroups gg{};
    int nblk = 0;
    for (; i < n && gg.n < kMaxGemmGroups; ++i) {
      GemmParams q = ps[i];
      set_tiles<EPI, NB>(q);
      const int tiles = q.tiles_m * q.tiles_n;
      if (tiles == 0) continue;
      gg.p[gg.n] = q;
      gg.start[gg.n] = nblk;
      nblk += (tiles + 7) / 8 * 8;
      ++gg.n;
    }
    gg.start[gg.n] = nblk;
    if (gg.n == 0) continue;
    if constexpr (kGrouped8<EPI, NB>)
      hipLaunchKernelGGL((gemm8_grouped_kernel<NN, EPI, QRB>), dim3(nblk), dim3(NT8), 0, stream, gg);
    else
      hipLaunchKernelGGL((gemm_bf16_grouped_kernel<NN, EPI, QRB, NB>), dim3(nblk), dim3(NTHREADS), 0, stream, gg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Parameter tables reach the device through a pinned host ring (one per
// device, created on first use and kept until the process ends): the host
// writes a table into a region of the ring, and one workgroup on the stream
// (fetch_table_kernel) reads it from host memory into the device table, then
// stores the region's tag into that region's completion slot, also in pinned
// host memory. So the table moves in stream order with no copy engine and no
// event: a copy handed to the DMA engine makes the next kernel on the stream
// wait for a cross-engine signal, about 20 microseconds each on MI355X. A
// region is written again only once every earlier use it overlaps shows its
// tag in its slot; the host never waits for it. `done` stays false when such
// a use is still pending, when the stream is being captured into a graph, or
// when the table is larger than the ring: the caller then writes the table
// with copy kernels on the stream.
constexpr size_t kStageBytes = size_t(16) << 20;
constexpr size_t kStageAlign = 256;
constexpr size_t kStageSlots = kStageBytes / kStageAlign;  // one per possible region start

static_assert(kStageSlots <= 65536, "slot index in 16 bits");

// Workgroup w of the fetch copies words [w * per, (w + 1) * per) of the
// table (the last also the 4-byte tail) and then marks slot w of the use.
__global__ __launch_bounds__(256) void fetch_table_kernel(const uint64_t* src, uint64_t* dst, int64_t n8, int64_t per,
                                                          const uint32_t* src_tail, uint32_t* dst_tail,
                                                          uint64_t* slots, uint64_t tag) {
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n8 ? lo + per : n8;
  // system-scope loads: the ring is host memory the host rewrites between
  // uses, so no cached copy of an earlier use may serve them
  for (int64_t i = lo + threadIdx.x; i < hi; i += 8 * 256) {
    uint64_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t j = i + int64_t(k) * 256;
      v[k] = j < hi ? __hip_atomic_load(src + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t j = i + int64_t(k) * 256;
      if (j < hi) dst[j] = v[k];
    }
  }
  if (src_tail != nullptr && blockIdx.x + 1 == gridDim.x && threadIdx.x == 0)
    *dst_tail = __hip_atomic_load(src_tail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  // every thread's loads have returned (their values were stored above); the
  // mark only tells the host the region was read, so it needs no release
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(slots + blockIdx.x, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

struct TableStage {
  char* host = nullptr;       // ring, then kStageSlots completion slots
  char* dev = nullptr;        // the same memory as the device addresses it
  uint64_t next_tag = 1;
  StageRing<uint64_t> ring{kStageBytes};
};
std::mutex g_stage_mu;
std::map<int, TableStage> g_stage;

static hipError_t stage_table(const void* src, size_t bytes, void* dst, hipStream_t st, bool& done) {
  done = false;
  if (bytes > kStageBytes || bytes % 4 || reinterpret_cast<uintptr_t>(dst) % 8) return hipSuccess;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) return hipSuccess;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_stage_mu);
  TableStage& S = g_stage[dev];
  if (!S.host) {
    const size_t total = kStageBytes + kStageSlots * sizeof(uint64_t);
    void* d = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&S.host), total, hipHostMallocDefault) != hipSuccess ||
        hipHostGetDevicePointer(&d, S.host, 0) != hipSuccess) {
      if (S.host) (void)hipHostFree(S.host);
      S.host = nullptr;
      (void)hipGetLastError();
      return hipSuccess;  // no staging memory: copy kernels
    }
    std::memset(S.host + kStageBytes, 0, kStageSlots * sizeof(uint64_t));
    S.dev = static_cast<char*>(d);
  }
  volatile uint64_t* slots = reinterpret_cast<volatile uint64_t*>(S.host + kStageBytes);
  const size_t len = (bytes + kStageAlign - 1) / kStageAlign * kStageAlign;
  // one workgroup per 16 KB (at most 64), each marking its own slot: the
  // slots of a use are those of its own 256-byte blocks, so live uses never
  // share one
  const int64_t n8 = static_cast<int64_t>(bytes / 8);
  int nwg = static_cast<int>((bytes + 16383) / 16384);
  nwg = std::max(1, std::min({nwg, 64, static_cast<int>(len / kStageAlign)}));
  const int64_t per = (n8 + nwg - 1) / nwg;
  size_t off = 0;
  // a use is packed as tag << 22 | workgroups << 16 | first slot
  const int got = S.ring.acquire(len, off, [slots](uint64_t ev) {
    const uint64_t first = ev & 0xffff, cnt = (ev >> 16) & 0x3f, tg = ev >> 22;
    for (uint64_t w = 0; w <= cnt; ++w)
      if (slots[first + w] != tg) return 0;
    return 1;
  });
  uint64_t spent = 0;
  while (S.ring.take_spare(spent)) {
  }
  if (got <= 0) return hipSuccess;
  std::memcpy(S.host + off, src, bytes);
  const uint64_t slot = off / kStageAlign;
  const uint64_t tag = S.next_tag++;
  const bool tail = bytes % 8 != 0;
  hipLaunchKernelGGL(fetch_table_kernel, dim3(nwg), dim3(256), 0, st,
                     reinterpret_cast<const uint64_t*>(S.dev + off), static_cast<uint64_t*>(dst), n8, per,
                     tail ? reinterpret_cast<const uint32_t*>(S.dev + off + bytes - 4) : nullptr,
                     tail ? reinterpret_cast<uint32_t*>(static_cast<char*>(dst) + bytes - 4) : nullptr,
                     reinterpret_cast<uint64_t*>(S.dev + kStageBytes) + slot, tag);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  S.ring.commit(off, len, tag << 22 | uint64_t(nwg - 1) << 16 | slot);
  done = true;
  return hipSuccess;
}

template <bool NN, int EPI, int QRB = 0, int NB = 8>
static hipError_t launch_table_t(const GemmParams* ps, int n, GemmParams* table, hipStream_t stream,
                                 TableBatch* batch) {
  for (int i0 = 0; i0 < n; i0 += kMaxTableGroups) {
    const int cnt = n - i0 < kMaxTableGroups ? n - i0 : kMaxTableGroups;
    GroupStarts gs{};
    int nblk = 0;
    std::vector<GemmParams> qs(ps + i0, ps + i0 + cnt);
    int maxt = 0;
    for (int i = 0; i < cnt; ++i) {
      set_tiles<EPI, NB>(qs[i]);
      maxt = std::max(maxt, qs[i].tiles_m * qs[i].tiles_n);
    }
    // pinned when there are many groups and each fits about two waves of one
    // XCD's 32 compute units; else every group spread over the eight XCDs
    gs.pinned = cnt >= 16 && maxt <= 64;
    if (gs.pinned) {
      // longest groups first, each to the XCD with the fewest slots so far
      std::vector<int> ord(cnt), xcd(cnt);
      for (int i = 0; i < cnt; ++i) ord[i] = i;
      std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
        return qs[a].tiles_m * qs[a].tiles_n > qs[b].tiles_m * qs[b].tiles_n;
      });
      int load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int i : ord) {
        const int x = static_cast<int>(std::min_element(load, load + 8) - load);
        xcd[i] = x;
        load[x] += qs[i].tiles_m * qs[i].tiles_n;
      }
      std::vector<GemmParams> by;
      by.reserve(cnt);
      int k = 0;
      for (int x = 0; x < 8; ++x) {
        gs.xfirst[x] = k;
        int slot = 0;
        for (int i : ord) {
          if (xcd[i] != x) continue;
          by.push_back(qs[i]);
          gs.start[k++] = slot;
          slot += qs[i].tiles_m * qs[i].tiles_n;
        }
      }
      gs.xfirst[8] = k;
      qs.swap(by);
      nblk = 8 * *std::max_element(load, load + 8);
    } else {
      for (int i = 0; i < cnt; ++i) {
        gs.start[i] = nblk;
        nblk += (qs[i].tiles_m * qs[i].tiles_n + 7) / 8 * 8;
      }
    }
    if (!gs.pinned) gs.start[cnt] = nblk;
    gs.n = cnt;
    if (nblk == 0) continue;
    if (batch) {
      const size_t bytes = qs.size() * sizeof(GemmParams);
      void* dt = batch->add(qs.data(), bytes);
      if (!dt) {
        const hipError_t me = batch->make_room();
        if (me != hipSuccess) return me;
        dt = batch->add(qs.data(), bytes);
        if (!dt) return hipErrorInvalidValue;  // larger than the whole batch
      }
      const GemmParams* tp = static_cast<const GemmParams*>(dt);
      batch->defer([tp, gs, nblk, stream]() -> hipError_t {
        launch_table_kernel<NN, EPI, QRB, NB>(tp, gs, nblk, stream);
        return hipGetLastError();
      });
      continue;
    }
    bool staged = false;
    hipError_t se = stage_table(qs.data(), qs.size() * sizeof(GemmParams), table, stream, staged);
    if (se != hipSuccess) return se;
    for (int i = 0; !staged && i < cnt; i += kMaxGemmGroups) {  // copy kernels, kMaxGemmGroups blocks each
      TableChunk tc{};
      tc.n = cnt - i < kMaxGemmGroups ? cnt - i : kMaxGemmGroups;
      for (int j = 0; j < tc.n; ++j) tc.p[j] = qs[i + j];
      tc.dst = table + i;
      hipLaunchKernelGGL(write_table_kernel, dim3(1), dim3(256), 0, stream, tc);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    launch_table_kernel<NN, EPI, QRB, NB>(table, gs, nblk, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {
// copy kernel of stage_device_table: up to 3.5 KB of words per launch, in
// its arguments
struct WordChunk {
  uint32_t w[896];
  uint32_t* dst;
  int32_t n;
};
__global__ __launch_bounds__(256) void write_words_kernel(WordChunk c) {
  for (int i = threadIdx.x; i < c.n; i += blockDim.x) c.dst[i] = c.w[i];
}

}  // namespace

hipError_t stage_device_table(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 4) return hipErrorInvalidValue;
  bool staged = false;
  const hipError_t se = stage_table(src, bytes, dst, stream, staged);
  if (se != hipSuccess || staged) return se;
  const uint32_t* s = static_cast<const uint32_t*>(src);
  uint32_t* d = static_cast<uint32_t*>(dst);
  const size_t n = bytes / 4;
  for (size_t i = 0; i < n; i += 896) {
    WordChunk c;
    c.n = static_cast<int32_t>(n - i < 896 ? n - i : 896);
    std::memcpy(c.w, s + i, size_t(c.n) * 4);
    c.dst = d + i;
    hipLaunchKernelGGL(write_words_kernel, dim3(1), dim3(256), 0, stream, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool NN, int EPI, int QRB = 0>
static hipError_t launch8q4_t(GemmParams p, hipStream_t stream) {
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  p.tiles_n = EPI == EPI_SWIGLU_FWD ? static_cast<int>((p.N + BN / 2 - 1) / (BN / 2))
                                    : static_cast<int>((p.N + BN - 1) / BN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
  const int nblk = p.tiles_m * p.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm8q4_kernel<NN, EPI, QRB>), dim3(nblk), dim3(NT8), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_q4(const GemmParams& p, int nn, int epi, hipStream_t stream) {
  if (p.tile_n != 0 && p.tile_n != 256) return hipErrorInvalidValue;  // 256-wide tiles only
  // one or two leading 4-bit segments, the rest dense
  if (p.nseg < 1 || !p.seg[0].bint4 || (p.nseg > 2 && p.seg[2].bint4)) return hipErrorInvalidValue;
  if (!nn && epi == EPI_STORE) return launch8q4_t<false, EPI_STORE>(p, stream);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch8q4_t<false, EPI_SWIGLU_FWD>(p, stream);
  if (nn && epi == EPI_STORE) return launch8q4_t<true, EPI_STORE>(p, stream);
  if (nn && epi == EPI_SWIGLU_BWD) {
    if (p.pj_part0 == nullptr) return launch8q4_t<true, EPI_SWIGLU_BWD, 0>(p, stream);
    if (p.pj_r16 == 16) return launch8q4_t<true, EPI_SWIGLU_BWD, 1>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16(const GemmParams& p, int nn, int epi, hipStream_t stream) {
  if (epi == EPI_STORE && p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
  const bool narrow_store = epi == EPI_STORE && p.tile_n == 128;  // 256 x 128 tiles for narrow products
  // eight-wave ping-pong where it measured faster (gate/up, and dZ without
  // the fused rank products); the plain products keep four waves
  if (!nn && epi == EPI_STORE)
    return narrow_store ? launch_t<false, EPI_STORE, 0, 4>(p, stream) : launch_t<false, EPI_STORE>(p, stream);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch8_t<false, EPI_SWIGLU_FWD>(p, stream);
  if (nn && epi == EPI_STORE)
    return narrow_store ? launch_t<true, EPI_STORE, 0, 4>(p, stream) : launch_t<true, EPI_STORE>(p, stream);
  if (nn && epi == EPI_SWIGLU_BWD) {
    const bool narrow = p.tile_n == 128;
    if (p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
    if (p.pj_part0 == nullptr)
      return narrow ? launch_t<true, EPI_SWIGLU_BWD, 0, 4>(p, stream) : launch8_t<true, EPI_SWIGLU_BWD, 0>(p, stream);
    if (p.pj_r16 == 16)
      return narrow ? launch_t<true, EPI_SWIGLU_BWD, 1, 4>(p, stream) : launch8_t<true, EPI_SWIGLU_BWD, 1>(p, stream);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16_grouped(const GemmParams* ps, int n, int nn, int epi, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const GemmParams& p = ps[0];  // every product of one call is of one kind
  if (!nn && epi == EPI_STORE) return launch_grouped_t<false, EPI_STORE>(ps, n, stream);
  if (epi == EPI_STORE_F32) {  // split-K partials: 256 x 256 tiles, N a multiple of 4
    for (int i = 0; i < n; ++i)
      if ((ps[i].tile_n != 0 && ps[i].tile_n != 256) || ps[i].N % 4 || ps[i].ldc % 4) return hipErrorInvalidValue;
    return nn ? launch_grouped_t<true, EPI_STORE_F32>(ps, n, stream) : launch_grouped_t<false, EPI_STORE_F32>(ps, n, stream);
  }
  if (!nn && epi == EPI_SWIGLU_FWD) return launch_grouped_t<false, EPI_SWIGLU_FWD>(ps, n, stream);
  if (nn && epi == EPI_STORE) return launch_grouped_t<true, EPI_STORE>(ps, n, stream);
  if (nn && epi == EPI_SWIGLU_BWD) {
    const bool narrow = p.tile_n == 128;
    if (p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
    if (p.pj_part0 == nullptr)
      return narrow ? launch_grouped_t<true, EPI_SWIGLU_BWD, 0, 4>(ps, n, stream)
                    : launch_grouped_t<true, EPI_SWIGLU_BWD, 0, 8>(ps, n, stream);
    if (p.pj_r16 == 16)
      return narrow ? launch_grouped_t<true, EPI_SWIGLU_BWD, 1, 4>(ps, n, stream)
                    : launch_grouped_t<true, EPI_SWIGLU_BWD, 1, 8>(ps, n, stream);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16_grouped_table(const GemmParams* ps, int n, int nn, int epi, GemmParams* table,
                                          hipStream_t stream, TableBatch* batch) {
  if (n <= 0) return hipSuccess;
  const GemmParams& p = ps[0];
  if (epi == EPI_STORE_F32) {  // split-K partials: 256 x 256 tiles, N a multiple of 4
    for (int i = 0; i < n; ++i)
      if ((ps[i].tile_n != 0 && ps[i].tile_n != 256) || ps[i].N % 4 || ps[i].ldc % 4) return hipErrorInvalidValue;
    return nn ? launch_table_t<true, EPI_STORE_F32>(ps, n, table, stream, batch)
              : launch_table_t<false, EPI_STORE_F32>(ps, n, table, stream, batch);
  }
  if (!nn && epi == EPI_STORE) return launch_table_t<false, EPI_STORE>(ps, n, table, stream, batch);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch_table_t<false, EPI_SWIGLU_FWD>(ps, n, table, stream, batch);
  if (nn && epi == EPI_STORE) return launch_table_t<true, EPI_STORE>(ps, n, table, stream, batch);
  if (nn && epi == EPI_SWIGLU_BWD) {
    const bool narrow = p.tile_n == 128;
    if (p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
    if (p.pj_part0 == nullptr)
      return narrow ? launch_table_t<true, EPI_SWIGLU_BWD, 0, 4>(ps, n, table, stream, batch)
                    : launch_table_t<true, EPI_SWIGLU_BWD, 0, 8>(ps, n, table, stream, batch);
    if (p.pj_r16 == 16)
      return narrow ? launch_table_t<true, EPI_SWIGLU_BWD, 1, 4>(ps, n, table, stream, batch)
                    : launch_table_t<true, EPI_SWIGLU_BWD, 1, 8>(ps, n, table, stream, batch);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace lmlp
