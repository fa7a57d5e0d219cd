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

#include <cstring>
#include <deque>
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
template <int CHUNKS>
__device__ __forceinline__ void lds_rows_to_global(const char* lds, int pitch, int rows, bf16_t* dst,
                                                   int64_t ldc, uint32_t m_rows, int64_t ncols) {
  const int tid = threadIdx.x;
  const int chunk = tid % CHUNKS;
  const int rsub = tid / CHUNKS;
  constexpr int RSTEP = NTHREADS / CHUNKS;
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
struct EpiPre {
  uint4 rk[10];
};

template <int EPI, int QRB>
__device__ __forceinline__ void epi_preload(const GemmParams& p, const TileCtx& t, EpiPre& pre) {
  if (EPI != EPI_SWIGLU_BWD || QRB != 1) return;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    const int idx = tid + NTHREADS * (j < 4 ? j : j - 4);
    const int row = idx >> 5, c = idx & 31;
    const bf16_t* src;
    bool ok;
    if (j < 4) {
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

// NB: 16-column blocks per wave (8: 256-wide tiles; 4: 128-wide, the plain
// and backward epilogues only, with the upper half of the staging left idle).
template <int EPI, int QRB = 0, int NB = 8>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, f32x4_t (&acc)[8][NB], const TileCtx& t,
                                             int wm, int wn, char* smem, const EpiPre& pre) {
  static_assert(NB == 8 || EPI != EPI_SWIGLU_FWD, "gate/up tiles are 256 wide");
  const int lrow = t.lane & 15;
  const int lcol = 4 * (t.lane >> 4);
  if (EPI == EPI_STORE) {
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
    lds_rows_to_global<32>(smem, EP_PITCH_C, 256, C, p.ldc, t.m_rows, t.n_rows);
  } else if (EPI == EPI_SWIGLU_FWD) {
    // tiles (a, 2q) hold G and (a, 2q+1) hold U of gate/up columns
    // j0 + wn*64 + 16q + lcol .. +3; both go to LDS rounded to bf16, then one
    // pass per row chunk stores G and U and forms Z = SiLU(G) U from the same
    // rounded values
    char* gbuf = smem;
    char* ubuf = smem + 256 * EP_PITCH_GU;
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int off = (wm * 128 + a * 16 + lrow) * EP_PITCH_GU + (wn * 64 + q * 16 + lcol) * 2;
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
    for (int r = rsub; r < 256; r += NTHREADS / 16) {
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
    // thread -> 8 consecutive columns (chunk) of rows rsub, rsub + 8, ... of a half
    const int tid = threadIdx.x;
    const int chunk = tid & 31;
    const int rsub = tid >> 5;
    const bool cval = static_cast<uint32_t>(chunk * 8) < t.n_rows;
    // G and U of one half-tile (16 rows per thread), fetched before they are
    // needed; invalid positions read element 0 and are never stored
    uint4 gv[16], uv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * i + rsub;
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
      for (int i = 0; i < 16; ++i) {
        const int rl = 8 * i + rsub;  // row within the half
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
    constexpr int JB = NB / 2;  // 16-column blocks of column products per wave
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
    for (int j = 0; j < 10; ++j) {
      const int idx = tid + NTHREADS * (j < 4 ? j : j - 4);
      const int row = idx >> 5, c = idx & 31;
      char* dst = (j < 4 ? bt : pt) + row * 512 + ((c ^ (row & 7)) << 4);
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
    constexpr int CH = 4 * NB;         // 16-byte chunks of a staging row
    constexpr int RS = NTHREADS / CH;  // staging rows per step
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
      // (B_g^T row n = l & 15), likewise Q_u: wave w takes token block w & 1 of
      // the pass and product w >> 1; the staged chunk (row l & 15, chunk
      // 4 ks + l / 16) is the MFMA source as it stands.
      {
        const int tb = t.wave & 1;
        const int pr = t.wave >> 1;
        const char* src = (pr ? sub : sgb) + (tb * 16 + lrow) * EP_SP;
        const char* brow = bt + (pr * 16 + lrow) * 512;
        f32x4_t q = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NB; ++ks) {
          const int ch = ks * 4 + lch;
          const uint4 bv = *reinterpret_cast<const uint4*>(brow + ((ch ^ (lrow & 7)) << 4));
          q = mma<bf16_t>::step(bv, *reinterpret_cast<const uint4*>(src + ch * 16), q);
        }
        // lane l holds Q[token = staging row 16 tb + (l & 15)][n = 4 (l >> 4) .. +3]:
        // one split-K slice (this tile column)
        const int r = tb * 128 + 16 * a + lrow;
        if (static_cast<uint32_t>(r) < t.m_rows) {
          const int64_t base = ((p.pj_slice0 + t.n0 / (32 * NB)) * p.pj_T + t.m0 + r) * 16 + 4 * lch;
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
  EpiPre pre;
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

// ---- 4-bit B operand (NT products with 4-bit block weights) ---------------
// The weight panel arrives as codes and scales and is decoded in LDS:
//  * ring stage (24 KB): the A tile (16 KB, as in the dense kernel); the codes
//    [256 packed rows][16 bytes] (one DMA per wave, lane = row); the fp32
//    scales of the k-tile's 64-block, one 1 KB slot per wave (64 rows, lanes
//    0-15 carry four rows each, the rest of the slot reads zero).
//  * two decoded B tiles (16 KB each, the dense K-major layout) outside the
//    ring. During k-tile kt every thread decodes one packed row of tile kt+2
//    (a row its own wave fetched, so only its own vmcnt wait is needed) into
//    buffer kt & 1, while the waves read tile kt+1's B fragments from buffer
//    (kt + 1) & 1; the barrier of tile kt+1 publishes the decoded rows.
//    Each packed row is decoded once per workgroup (decoding inside the
//    fragment reads would repeat it in both waves of a B half; measured
//    about 8% slower at the Llama-3-8B shapes).
// Packed row order: gate/up tiles hold gate rows j0 .. j0+127 in packed rows
// 0-127 and the up rows in 128-255 (waves 0-1 fetch gate, 2-3 up); the
// decoded tile interleaves them every 16 rows as the dense kernel does.
// Decoding is the block rule of the 4-bit format: w = bf16_rne(q * scale),
// exact in fp32 before the one rounding (dq_chunk).
// The adapter segment (dense bf16) follows the 4-bit loop as a short
// unpipelined tail.
constexpr int Q4_CODES = TILE_BYTES;             // offset of the codes in a stage
constexpr int Q4_SCALES = TILE_BYTES + 4096;     // offset of the scale slots
constexpr int Q4_STAGE = TILE_BYTES + 8192;      // 24 KB
constexpr int Q4_STAGES = 5;
constexpr int Q4_DEC = Q4_STAGES * Q4_STAGE;     // decoded B tiles start here
constexpr int Q4_LDS0 = Q4_DEC + 2 * TILE_BYTES;  // 152 KB
constexpr int Q4_LDS = Q4_LDS0 > EP_LDS_BYTES ? Q4_LDS0 : EP_LDS_BYTES;

struct Q4Dma {
  rsrc_t rA;            // activation panel of this tile row block
  uint32_t offA[4];
  uint32_t lda_b;
  const char* codes;    // first packed row of this wave's 64 rows
  uint32_t ldq_b;       // bytes per packed row (K / 2)
  uint32_t qrows;       // valid rows of this wave's 64 (0 or 64)
  const char* scales;   // fp32 [K/64][N] at this wave's first row
  uint32_t ld_sc_b;     // bytes per scale block row (N * 4)
  int k0, kt;
};

template <int EPI>
__device__ __forceinline__ void q4_dma_init(Q4Dma& d, const GemmParams& p, const TileCtx& t) {
  const GemmSeg& g = p.seg[0];
  d.lda_b = static_cast<uint32_t>(g.lda * 2);
  d.rA = make_rsrc(static_cast<const char*>(g.a) + t.m0 * d.lda_b, t.m_rows * d.lda_b);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d.offA[i] = static_cast<uint32_t>(64 * t.wave + 16 * i + (t.lane >> 2)) * d.lda_b + (t.c1 << 4);
  d.ldq_b = static_cast<uint32_t>(g.ldb / 2);
  const bool up = EPI == EPI_SWIGLU_FWD && t.wave >= 2;
  const int64_t row0 = EPI == EPI_SWIGLU_FWD ? t.j0 + 64 * (t.wave & 1) : t.n0 + 64 * t.wave;
  d.qrows = row0 < p.N ? 64u : 0u;  // N and row0 are multiples of 64
  d.codes = static_cast<const char*>(up ? g.b1 : g.b0) + row0 * d.ldq_b;
  d.scales = static_cast<const char*>(up ? g.bs1 : g.bs0) + row0 * 4;
  d.ld_sc_b = static_cast<uint32_t>(p.N * 4);
  d.k0 = 0;
  d.kt = 0;
}

// DMA instruction j (0..5) of k-tile d.kt into stage `st`: 0-3 the A tile,
// 4 the codes, 5 the scales. Past the last 4-bit k-tile everything reads zero.
__device__ __forceinline__ void q4_dma_issue(const Q4Dma& d, int j, char* st, int nkq, const TileCtx& t) {
  const bool live = d.kt < nkq;
  if (j < 4) {
    dma16(d.rA, st + (64 * t.wave + 16 * j) * 64, live ? d.offA[j] : OOB, d.k0 * 2);
  } else if (j == 4) {
    const rsrc_t r = make_rsrc(d.codes, (live ? d.qrows : 0u) * d.ldq_b);
    dma16(r, st + Q4_CODES + t.wave * 1024, static_cast<uint32_t>(t.lane) * d.ldq_b, d.k0 / 2);
  } else {
    // the 64-block of this k-tile: one descriptor per block row, so the
    // range check covers exactly this wave's 64 scales
    const rsrc_t r = make_rsrc(d.scales + static_cast<int64_t>(d.k0 / 64) * d.ld_sc_b, live ? d.qrows * 4 : 0u);
    dma16(r, st + Q4_SCALES + t.wave * 1024, t.lane < 16 ? static_cast<uint32_t>(t.lane) * 16 : OOB, 0);
  }
}

__device__ __forceinline__ void q4_dma_advance(Q4Dma& d) {
  ++d.kt;
  d.k0 += BK;
}

// decoded-tile row of packed row pr (gate/up: interleave the two panels)
template <int EPI>
__device__ __forceinline__ int q4_dense_row(int pr) {
  if (EPI != EPI_SWIGLU_FWD) return pr;
  const int panel = pr >> 7, r = pr & 127;
  return (r >> 4) * 32 + panel * 16 + (r & 15);
}

// decode chunk c (8 codes) of this thread's packed row into the decoded tile
template <int EPI>
__device__ __forceinline__ void q4_decode_chunk(char* dec, int c, uint32_t codes, float sc, int drow) {
  *reinterpret_cast<uint4*>(dec + drow * 64 + ((c ^ ((drow >> 1) & 3)) << 4)) = dq_chunk(codes, sc);
}

__device__ __forceinline__ uint4 read_bq(const ReadCtx& rc, const char* dec, int b) {
  return *reinterpret_cast<const uint4*>(dec + rc.rdB + b * 1024);
}

// One 4-bit k-tile kt (stage st_cur, decoded B fragments already in fb).
template <int EPI>
__device__ __forceinline__ void q4_tile(f32x4_t (&acc)[8][8], uint4 (&fa)[8], const uint4 (&fb)[8],
                                        uint4 (&fbn)[8], Q4Dma& d, int& st_cur, char* smem, const ReadCtx& rc,
                                        const TileCtx& t, int nkq, int kt) {
  const int st_nxt = st_cur + 1 == Q4_STAGES ? 0 : st_cur + 1;
  const int st_dma = st_cur == 0 ? Q4_STAGES - 1 : st_cur - 1;  // tile kt-1's stage
  const int st_dec = st_nxt + 1 == Q4_STAGES ? 0 : st_nxt + 1;  // tile kt+2's stage
  const char* nxt = smem + st_nxt * Q4_STAGE;
  char* dbuf = smem + st_dma * Q4_STAGE;
  char* dec_w = smem + Q4_DEC + (kt & 1) * TILE_BYTES;              // tile kt+2, decoded now
  const char* dec_r = smem + Q4_DEC + ((kt + 1) & 1) * TILE_BYTES;  // tile kt+1
  mfma_group<8>(acc, 0, fa, fb);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<6>();  // tiles kt+1 and kt+2 landed (this wave); kt+3 may fly
  __syncthreads();
  const int pr = 64 * t.wave + t.lane;
  const char* qsrc = smem + st_dec * Q4_STAGE + Q4_CODES + pr * 16;
  const char* ssrc = smem + st_dec * Q4_STAGE + Q4_SCALES + t.wave * 1024 + t.lane * 4;
#pragma unroll
  for (int g = 1; g < 8; ++g) {
    mfma_group<8>(acc, g, fa, fb);
    __builtin_amdgcn_sched_barrier(0);
    if (g <= 6) q4_dma_issue(d, g - 1, dbuf, nkq, t);
    fa[g - 1] = read_a(rc, nxt, g - 1);
    if (g <= 4) {
      fbn[2 * g - 2] = read_bq(rc, dec_r, 2 * g - 2);
      fbn[2 * g - 1] = read_bq(rc, dec_r, 2 * g - 1);
    }
    if (g >= 2 && g <= 5)
      q4_decode_chunk<EPI>(dec_w, g - 2, *reinterpret_cast<const uint32_t*>(qsrc + 4 * (g - 2)),
                           *reinterpret_cast<const float*>(ssrc), q4_dense_row<EPI>(pr));
    __builtin_amdgcn_sched_barrier(0);
  }
  q4_dma_advance(d);
  fa[7] = read_a(rc, nxt, 7);
  __builtin_amdgcn_sched_barrier(0);
  st_cur = st_nxt;
}

template <int EPI>
__device__ __forceinline__ void gemm_q4_body(const GemmParams& p) {
  __shared__ __attribute__((aligned(1024))) char smem[Q4_LDS];

  TileCtx t;
  t.lane = threadIdx.x & 63;
  t.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.c1 = (t.lane & 3) ^ ((t.lane >> 3) & 3);
  const int wm = t.wave >> 1;
  const int wn = t.wave & 1;
  select_tile<EPI>(p, t, blockIdx.x, gridDim.x);

  const int nkq = static_cast<int>(p.seg[0].K / BK);  // K is a multiple of 64: an even count

  f32x4_t acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = t.lane & 15;
  const int lgrp = t.lane >> 4;
  ReadCtx rc;
  rc.rdA = static_cast<uint32_t>((wm * 128 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.rdB = static_cast<uint32_t>((wn * 128 + lrow) * 64 + ((lgrp ^ ((lrow >> 1) & 3)) << 4));
  rc.nsw = 0;
  rc.rdN = 0;

  // ---- prologue: DMA of tiles 0-3, decode of tiles 0 and 1
  Q4Dma d;
  q4_dma_init<EPI>(d, p, t);
#pragma unroll
  for (int s = 0; s < Q4_STAGES - 1; ++s) {
#pragma unroll
    for (int j = 0; j < 6; ++j) q4_dma_issue(d, j, smem + s * Q4_STAGE, nkq, t);
    q4_dma_advance(d);
  }
  wait_vmcnt<6>();  // tiles 0-2 landed (this wave)
  {
    const int pr = 64 * t.wave + t.lane;
    const int drow = q4_dense_row<EPI>(pr);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 codes = *reinterpret_cast<const uint4*>(smem + s * Q4_STAGE + Q4_CODES + pr * 16);
      const float sc = *reinterpret_cast<const float*>(smem + s * Q4_STAGE + Q4_SCALES + t.wave * 1024 + t.lane * 4);
      char* dec = smem + Q4_DEC + s * TILE_BYTES;
      q4_decode_chunk<EPI>(dec, 0, codes.x, sc, drow);
      q4_decode_chunk<EPI>(dec, 1, codes.y, sc, drow);
      q4_decode_chunk<EPI>(dec, 2, codes.z, sc, drow);
      q4_decode_chunk<EPI>(dec, 3, codes.w, sc, drow);
    }
  }
  __syncthreads();
  uint4 fa[8], fbA[8], fbB[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) fbA[b] = read_bq(rc, smem + Q4_DEC, b);
#pragma unroll
  for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, smem, a);

  int st_cur = 0;
  // one k-tile per trip: with the decode in the groups, a two-tile body
  // makes the register allocator shuffle the accumulators every trip; the
  // copy of the next B fragments (32 moves) is the cheaper price
  for (int kt = 0; kt < nkq; ++kt) {
    q4_tile<EPI>(acc, fa, fbA, fbB, d, st_cur, smem, rc, t, nkq, kt);
#pragma unroll
    for (int b = 0; b < 8; ++b) fbA[b] = fbB[b];
  }
  wait_vmcnt<0>();

  // ---- adapter segment: dense bf16 k-tiles, one at a time
  if (p.nseg > 1 && p.seg[1].K > 0) {
    const Seg s1 = seg_at(p, 1);
    Dma da;
    da.seg = 1;
    da.kt = 0;
    da.k0 = 0;
    dma_load_seg<false, EPI>(da, s1, t);
    for (int k0 = 0; k0 < s1.K; k0 += BK) {
      __syncthreads();  // every wave is done with the LDS it is about to reuse
      da.k0 = k0;
#pragma unroll
      for (int j = 0; j < 8; ++j) dma_issue<false, EPI>(da, j, smem, 1, t);
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int b = 0; b < 8; ++b) fbA[b] = read_b<false>(rc, smem, b);
#pragma unroll
      for (int a = 0; a < 8; ++a) fa[a] = read_a(rc, smem, a);
#pragma unroll
      for (int g = 0; g < 8; ++g) mfma_group<8>(acc, g, fa, fbA);
    }
  }

  const EpiPre none{};
  epilogue_lds<EPI>(p, acc, t, wm, wn, smem, none);
}

template <int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_q4_kernel(GemmParams p) {
  gemm_q4_body<EPI>(p);
}

}  // namespace

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

// Groups whose parameter blocks sit in device memory (more groups than the
// kernel arguments hold): the same workgroup -> (group, tile) map, with the
// group starts in the arguments.
struct GroupStarts {
  int32_t start[kMaxTableGroups + 1];
  int32_t n;
};

template <bool NN, int EPI, int QRB, int NB>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_table_kernel(const GemmParams* __restrict__ table,
                                                                     GroupStarts gs) {
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  const int bid = blockIdx.x;
  int lo = 0, hi = gs.n - 1;  // the last group whose start is <= bid
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gs.start[mid] <= bid) lo = mid;
    else hi = mid - 1;
  }
  const GemmParams& p = table[lo];
  const int local = bid - gs.start[lo];
  const int tiles = p.tiles_m * p.tiles_n;
  if (local >= tiles) return;
  gemm_bf16_body<NN, EPI, QRB, NB>(p, local, tiles, smem);
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
  for (int i0 = 0; i0 < n; i0 += kMaxGemmGroups) {
    GemmGroups gg{};
    int nblk = 0;
    for (int i = i0; i < n && gg.n < kMaxGemmGroups; ++i) {
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
    hipLaunchKernelGGL((gemm_bf16_grouped_kernel<NN, EPI, QRB, NB>), dim3(nblk), dim3(NTHREADS), 0, stream, gg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Parameter tables reach the device through a pinned host ring and one copy
// on the stream (one per device, created on first use and kept until the
// process ends). A region of the ring is written again only after the event
// recorded behind its previous copy has completed. `done` stays false when
// the stream is being captured into a graph or the table is larger than the
// ring: the caller then writes the table with copy kernels.
constexpr size_t kStageBytes = size_t(4) << 20;
struct StageUse {
  size_t off, len;
  hipEvent_t ev;
};
struct TableStage {
  char* host = nullptr;
  size_t head = 0;
  std::deque<StageUse> inflight;  // in ring order: a new region can only overlap the oldest ones
  std::vector<hipEvent_t> spare;
};
std::mutex g_stage_mu;
std::map<int, TableStage> g_stage;

static hipError_t stage_table(const GemmParams* src, size_t bytes, GemmParams* dst, hipStream_t st, bool& done) {
  done = false;
  if (bytes > kStageBytes) return hipSuccess;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) return hipSuccess;
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_stage_mu);
  TableStage& S = g_stage[dev];
  if (!S.host && hipHostMalloc(reinterpret_cast<void**>(&S.host), kStageBytes, hipHostMallocDefault) != hipSuccess) {
    S.host = nullptr;
    (void)hipGetLastError();
    return hipSuccess;  // no staging memory: copy kernels
  }
  const size_t len = (bytes + 255) / 256 * 256;
  if (S.head + len > kStageBytes) S.head = 0;
  while (!S.inflight.empty()) {
    const StageUse& u = S.inflight.front();
    if (!(u.off < S.head + len && S.head < u.off + u.len)) break;
    e = hipEventSynchronize(u.ev);
    if (e != hipSuccess) return e;
    S.spare.push_back(u.ev);
    S.inflight.pop_front();
  }
  char* h = S.host + S.head;
  std::memcpy(h, src, bytes);
  e = hipMemcpyAsync(dst, h, bytes, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  hipEvent_t ev = nullptr;
  if (!S.spare.empty()) {
    ev = S.spare.back();
    S.spare.pop_back();
  } else {
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  e = hipEventRecord(ev, st);
  if (e != hipSuccess) return e;
  S.inflight.push_back({S.head, len, ev});
  S.head += len;
  done = true;
  return hipSuccess;
}

template <bool NN, int EPI, int QRB = 0, int NB = 8>
static hipError_t launch_table_t(const GemmParams* ps, int n, GemmParams* table, hipStream_t stream) {
  for (int i0 = 0; i0 < n; i0 += kMaxTableGroups) {
    const int cnt = n - i0 < kMaxTableGroups ? n - i0 : kMaxTableGroups;
    GroupStarts gs{};
    int nblk = 0;
    std::vector<GemmParams> qs(ps + i0, ps + i0 + cnt);
    for (int i = 0; i < cnt; ++i) {
      set_tiles<EPI, NB>(qs[i]);
      gs.start[i] = nblk;
      nblk += (qs[i].tiles_m * qs[i].tiles_n + 7) / 8 * 8;
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
    gs.start[cnt] = nblk;
    gs.n = cnt;
    if (nblk == 0) continue;
    hipLaunchKernelGGL((gemm_bf16_table_kernel<NN, EPI, QRB, NB>), dim3(nblk), dim3(NTHREADS), 0, stream,
                       static_cast<const GemmParams*>(table), gs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int EPI>
static hipError_t launch_q4(GemmParams p, hipStream_t stream) {
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  p.tiles_n = EPI == EPI_SWIGLU_FWD ? static_cast<int>((p.N + BN / 2 - 1) / (BN / 2))
                                    : static_cast<int>((p.N + BN - 1) / BN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
  const int nblk = p.tiles_m * p.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_q4_kernel<EPI>), dim3(nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_q4(const GemmParams& p, int epi, hipStream_t stream) {
  if (epi == EPI_STORE) return launch_q4<EPI_STORE>(p, stream);
  if (epi == EPI_SWIGLU_FWD) return launch_q4<EPI_SWIGLU_FWD>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16(const GemmParams& p, int nn, int epi, hipStream_t stream) {
  if (epi == EPI_STORE && p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
  const bool narrow_store = epi == EPI_STORE && p.tile_n == 128;  // 256 x 128 tiles for narrow products
  if (!nn && epi == EPI_STORE)
    return narrow_store ? launch_t<false, EPI_STORE, 0, 4>(p, stream) : launch_t<false, EPI_STORE>(p, stream);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch_t<false, EPI_SWIGLU_FWD>(p, stream);
  if (nn && epi == EPI_STORE)
    return narrow_store ? launch_t<true, EPI_STORE, 0, 4>(p, stream) : launch_t<true, EPI_STORE>(p, stream);
  if (nn && epi == EPI_SWIGLU_BWD) {
    const bool narrow = p.tile_n == 128;
    if (p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
    if (p.pj_part0 == nullptr)
      return narrow ? launch_t<true, EPI_SWIGLU_BWD, 0, 4>(p, stream) : launch_t<true, EPI_SWIGLU_BWD, 0, 8>(p, stream);
    if (p.pj_r16 == 16)
      return narrow ? launch_t<true, EPI_SWIGLU_BWD, 1, 4>(p, stream) : launch_t<true, EPI_SWIGLU_BWD, 1, 8>(p, stream);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16_grouped(const GemmParams* ps, int n, int nn, int epi, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const GemmParams& p = ps[0];  // every product of one call is of one kind
  if (!nn && epi == EPI_STORE) return launch_grouped_t<false, EPI_STORE>(ps, n, stream);
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
                                          hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const GemmParams& p = ps[0];
  if (!nn && epi == EPI_STORE) return launch_table_t<false, EPI_STORE>(ps, n, table, stream);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch_table_t<false, EPI_SWIGLU_FWD>(ps, n, table, stream);
  if (nn && epi == EPI_STORE) return launch_table_t<true, EPI_STORE>(ps, n, table, stream);
  if (nn && epi == EPI_SWIGLU_BWD) {
    const bool narrow = p.tile_n == 128;
    if (p.tile_n != 0 && p.tile_n != 128 && p.tile_n != 256) return hipErrorInvalidValue;
    if (p.pj_part0 == nullptr)
      return narrow ? launch_table_t<true, EPI_SWIGLU_BWD, 0, 4>(ps, n, table, stream)
                    : launch_table_t<true, EPI_SWIGLU_BWD, 0, 8>(ps, n, table, stream);
    if (p.pj_r16 == 16)
      return narrow ? launch_table_t<true, EPI_SWIGLU_BWD, 1, 4>(ps, n, table, stream)
                    : launch_table_t<true, EPI_SWIGLU_BWD, 1, 8>(ps, n, table, stream);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace lmlp
