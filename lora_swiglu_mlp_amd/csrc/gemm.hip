// fp32 MFMA GEMM with appended adapter K-steps and fused SwiGLU epilogues.
// (bf16 products run on the LDS-DMA kernels of gemm_bf16.hip; this
// register-staged kernel serves the fp32 dtype.)
//
// One kernel template serves the four large products of the fused LoRA MLP
// ("Unsloth 深度分析报告", section 创新之处):
//   gate/up  [G|U] = [X | sP] [Wg|Bg ; Wu|Bu]^T, epilogue Z = SiLU(G) * U   (NT)
//   down      Y    = [Z | sPd] [Wd | Bd]^T                                   (NT)
//   dZ        dZ   = [dY | sQd] [Wd ; Ad], epilogue dG, dU (SiLU' recompute) (NN)
//   dX        dX   = [dG | dU | sQ] [Wg ; Wu ; Agu]                         (NN)
// The rank-r adapter product is folded into the same K loop: the low-rank
// factor of the input side (s * X A^T, prepared by the row-projection kernel)
// is a short extra K segment of the A operand, and the matching B factor is
// the extra K segment of the B operand. So each output tile is finished in
// one pass, with the base and adapter terms summed in the same fp32
// accumulators.
//
// Tiling for gfx950: 256x256 output tile per 256-thread workgroup, 4 waves in
// a 2x2 grid, each wave 128x128 (8x8 MFMA 16x16 tiles, 256 fp32 accumulators
// per lane). K advances 128 bytes per tile (64 bf16 / 32 fp32); the A and B
// tiles are double-buffered in LDS (2 x 64 KB) with a 16-byte XOR swizzle.
// NN-layout B tiles (K rows, N contiguous) are transposed in registers
// between the global load and the LDS store, so the LDS image is always
// K-major and the MFMA operand reads are 16-byte and conflict-free.
#include "common.h"
#include "gemm_epilogue.h"
#include "kernels.h"

namespace lmlp {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int NTHREADS = 256;
constexpr int ROWCH = 8;  // 16-byte chunks per LDS row (128 bytes of K)

struct SegIter {
  int seg;
  int64_t k0;
};

template <typename T>
__device__ __forceinline__ SegIter locate(const GemmParams& p, int kt) {
  constexpr int BKE = ROWCH * elem<T>::CH;
  SegIter it{0, 0};
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s < p.nseg) {
      const int nk = static_cast<int>((p.seg[s].K + BKE - 1) / BKE);
      if (kt < nk) { it.seg = s; it.k0 = static_cast<int64_t>(kt) * BKE; return it; }
      kt -= nk;
    }
  }
  return it;
}

template <typename T, bool NN, int EPI>
struct Gemm {
  static constexpr int CH = elem<T>::CH;
  static constexpr int BKE = ROWCH * CH;

  // registers staged between the global load and the LDS store
  struct Stage {
    uint4 a[8];
    uint4 b[8];
  };

  __device__ static __forceinline__ void load_a(const GemmParams& p, const SegIter& it, int64_t m0,
                                                int tid, Stage& st) {
    const GemmSeg& sg = p.seg[it.seg];
    const T* A = static_cast<const T*>(sg.a);
    const int c = tid & 7;
    const int r = tid >> 3;
    const int64_t kc = it.k0 + c * CH;
    const bool kval = kc < sg.K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + r + 32 * i;
      if (kval && m < p.M)
        st.a[i] = *reinterpret_cast<const uint4*>(A + m * sg.lda + kc);
      else
        st.a[i] = zero4();
    }
  }

  // B operand, K-major source (NT). For the gate/up product the tile's rows
  // alternate in groups of 16 between the gate and the up weights, so that a
  // wave's neighbouring accumulator tiles hold G and U of the same (m, j).
  __device__ static __forceinline__ void load_b_nt(const GemmParams& p, const SegIter& it,
                                                   int64_t n0, int tid, Stage& st) {
    const GemmSeg& sg = p.seg[it.seg];
    const int c = tid & 7;
    const int r = tid >> 3;
    const T* B0 = static_cast<const T*>(sg.b0);
    const T* B1 = static_cast<const T*>(sg.b1);
    const int64_t kc = it.k0 + c * CH;
    const bool kval = kc < sg.K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = r + 32 * i;
      int64_t row;
      const T* Bp;
      if (EPI == EPI_SWIGLU_FWD) {
        const int q = rl >> 4;
        row = (n0 >> 1) + (q >> 1) * 16 + (rl & 15);
        Bp = (q & 1) ? B1 : B0;
      } else {
        row = n0 + rl;
        Bp = B0;
      }
      if (kval && row < p.N)
        st.b[i] = *reinterpret_cast<const uint4*>(Bp + row * sg.ldb + kc);
      else
        st.b[i] = zero4();
    }
  }

  // B operand, N-major source (NN): rows are K, N contiguous. Each thread
  // loads a CH x CH block (CH rows of K, one 16-byte chunk of N each) and
  // later writes it transposed.
  __device__ static __forceinline__ void load_b_nn(const GemmParams& p, const SegIter& it,
                                                   int64_t n0, int tid, Stage& st) {
    const GemmSeg& sg = p.seg[it.seg];
    constexpr int NB = BN / CH;          // column blocks per tile
    constexpr int BPT = (ROWCH * NB) / NTHREADS;  // blocks per thread
    const T* B = static_cast<const T*>(sg.b0);
#pragma unroll
    for (int bi = 0; bi < BPT; ++bi) {
      const int q = tid + NTHREADS * bi;
      const int nb = q % NB;
      const int kb = q / NB;
      const int64_t n = n0 + nb * CH;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int64_t k = it.k0 + kb * CH + i;
        if (k < sg.K && n < p.N)
          st.b[bi * CH + i] = *reinterpret_cast<const uint4*>(B + k * sg.ldb + n);
        else
          st.b[bi * CH + i] = zero4();
      }
    }
  }

  __device__ static __forceinline__ void store_a(uint4 (*As)[ROWCH], int tid, const Stage& st) {
    const int c = tid & 7;
    const int r = tid >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r + 32 * i;
      As[row][swz(row, c)] = st.a[i];
    }
  }

  __device__ static __forceinline__ void store_b(uint4 (*Bs)[ROWCH], int tid, const Stage& st) {
    if (!NN) {
      const int c = tid & 7;
      const int r = tid >> 3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = r + 32 * i;
        Bs[row][swz(row, c)] = st.b[i];
      }
      return;
    }
    constexpr int NB = BN / CH;
    constexpr int BPT = (ROWCH * NB) / NTHREADS;
#pragma unroll
    for (int bi = 0; bi < BPT; ++bi) {
      const int q = tid + NTHREADS * bi;
      const int nb = q % NB;
      const int kb = q / NB;
      const uint4* in = &st.b[bi * CH];
      if (CH == 8) {
        // 8x8 transpose of 16-bit values: out[j] collects element j of in[0..7]
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sh = (j & 1) * 16;
          auto pick = [&](const uint4& v) -> uint32_t {
            const uint32_t d = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
            return (d >> sh) & 0xFFFFu;
          };
          uint4 o;
          o.x = pick(in[0]) | (pick(in[1]) << 16);
          o.y = pick(in[2]) | (pick(in[3]) << 16);
          o.z = pick(in[4]) | (pick(in[5]) << 16);
          o.w = pick(in[6]) | (pick(in[7]) << 16);
          const int row = nb * CH + j;
          Bs[row][swz(row, kb)] = o;
        }
      } else {
        // 4x4 transpose of 32-bit values
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          auto pick = [&](const uint4& v) -> uint32_t {
            return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
          };
          uint4 o;
          o.x = pick(in[0]);
          o.y = pick(in[1]);
          o.z = pick(in[2]);
          o.w = pick(in[3]);
          const int row = nb * CH + j;
          Bs[row][swz(row, kb)] = o;
        }
      }
    }
  }

  __device__ static void run(const GemmParams& p) {
    __shared__ uint4 smem[2][2][BM][ROWCH];  // [buffer][A/B][row][chunk], 128 KB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    // ---- tile selection: XCD-aware, grouped along M
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    int logical = bid;
    {
      const int per = nblk / 8, rem = nblk % 8, x = bid % 8;
      logical = x * per + (x < rem ? x : rem) + bid / 8;
    }
    const int gm = p.group_m;
    const int width = gm * p.tiles_n;
    const int group = logical / width;
    const int first_m = group * gm;
    const int gsize = min(p.tiles_m - first_m, gm);
    const int tm = first_m + (logical % width) % gsize;
    const int tn = (logical % width) / gsize;
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;  // for SWIGLU_FWD: 2 * j0

    int nk = 0;
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < p.nseg) nk += static_cast<int>((p.seg[s].K + BKE - 1) / BKE);

    f32x4_t acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    Stage st;
    if (nk > 0) {
      SegIter it = locate<T>(p, 0);
      load_a(p, it, m0, tid, st);
      if (NN) load_b_nn(p, it, n0, tid, st); else load_b_nt(p, it, n0, tid, st);
      store_a(smem[0][0], tid, st);
      store_b(smem[0][1], tid, st);
    }
    __syncthreads();

    const int lrow = lane & 15;
    const int lch = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        SegIter it = locate<T>(p, kt + 1);
        load_a(p, it, m0, tid, st);
        if (NN) load_b_nn(p, it, n0, tid, st); else load_b_nt(p, it, n0, tid, st);
      }
      uint4 (*As)[ROWCH] = smem[buf][0];
      uint4 (*Bs)[ROWCH] = smem[buf][1];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = ks * 4 + lch;
        uint4 fa[8], fb[8];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const int row = wm * 128 + a * 16 + lrow;
          fa[a] = As[row][swz(row, ch)];
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int row = wn * 128 + b * 16 + lrow;
          fb[b] = Bs[row][swz(row, ch)];
        }
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[a][b] = mma<T>::step(fb[b], fa[a], acc[a][b]);
      }
      if (more) {
        store_a(smem[buf ^ 1][0], tid, st);
        store_b(smem[buf ^ 1][1], tid, st);
      }
      __syncthreads();
    }

    gemm_epilogue<T, EPI>(p, acc, m0, n0, wm, wn, lane);
  }
};

template <typename T, bool NN, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(GemmParams p) {
  Gemm<T, NN, EPI>::run(p);
}

}  // namespace

template <typename T, bool NN, int EPI>
static hipError_t launch_t(GemmParams p, hipStream_t stream) {
  p.tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  if (EPI == EPI_SWIGLU_FWD)
    p.tiles_n = static_cast<int>((p.N + BN / 2 - 1) / (BN / 2));
  else
    p.tiles_n = static_cast<int>((p.N + BN - 1) / BN);
  if (p.group_m <= 0) p.group_m = 8;
  if (p.group_m > p.tiles_m) p.group_m = p.tiles_m;
  const int nblk = p.tiles_m * p.tiles_n;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<T, NN, EPI>), dim3(nblk), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmParams& p, int nn, int epi, hipStream_t stream) {
  if (!nn && epi == EPI_STORE) return launch_t<float, false, EPI_STORE>(p, stream);
  if (!nn && epi == EPI_SWIGLU_FWD) return launch_t<float, false, EPI_SWIGLU_FWD>(p, stream);
  if (nn && epi == EPI_STORE) return launch_t<float, true, EPI_STORE>(p, stream);
  if (nn && epi == EPI_SWIGLU_BWD) return launch_t<float, true, EPI_SWIGLU_BWD>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace lmlp
