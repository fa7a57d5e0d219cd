// Epilogues of the MFMA GEMM (shared by the general and the bf16 kernels).
//
// Accumulator layout: acc[a][b] is the 16x16 output tile at rows
// wm*128 + 16a, columns wn*128 + 16b of the 256x256 workgroup tile, computed
// as D = SrcA * SrcB^T with the B fragment as SrcA, so lane l holds output row
// (l & 15) of the tile and 4 consecutive columns 4*(l >> 4) .. +3.
//   STORE       C = acc (dtype), rows < M, columns < N.
//   SWIGLU_FWD  tiles (a, 2q) and (a, 2q+1) are G and U of the same columns
//               j (the B rows alternate gate/up in groups of 16): store G and
//               U rounded to the dtype, and Z = SiLU(G) * U from the rounded
//               values (so backward recomputes exactly this Z).
//   SWIGLU_BWD  acc = dZ. Reload G and U, recompute sigmoid(G), SiLU(G) and
//               Z; dG = dZ * U * sig * (1 + G (1 - sig)), dU = dZ * SiLU(G).
//               This is the derivative of SiLU(g) * u: d/dg [g sig(g)] =
//               sig (1 + g (1 - sig)).
#pragma once

#include "common.h"
#include "kernels.h"

namespace lmlp {

template <typename T, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, f32x4_t (&acc)[8][8], int64_t m0,
                                              int64_t n0, int wm, int wn, int lane) {
  const int lrow = lane & 15;
  const int lcol = 4 * (lane >> 4);
  if (EPI == EPI_STORE) {
    T* C = static_cast<T*>(p.c0);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t m = m0 + wm * 128 + a * 16 + lrow;
      if (m >= p.M) continue;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t n = n0 + wn * 128 + b * 16 + lcol;
        if (n < p.N) store4(C + m * p.ldc + n, acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
      }
    }
  } else if (EPI == EPI_SWIGLU_FWD) {
    // tiles (a, 2q) hold G and (a, 2q+1) hold U for the same j
    T* Gp = static_cast<T*>(p.c0);
    T* Up = static_cast<T*>(p.c1);
    T* Zp = static_cast<T*>(p.c2);
    const int64_t j0 = n0 >> 1;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t m = m0 + wm * 128 + a * 16 + lrow;
      if (m >= p.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t j = j0 + wn * 64 + q * 16 + lcol;
        if (j >= p.N) continue;
        float g[4], u[4], z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g[i] = elem<T>::round(acc[a][2 * q][i]);
          u[i] = elem<T>::round(acc[a][2 * q + 1][i]);
          z[i] = g[i] * sigmoidf_fast(g[i]) * u[i];
        }
        const int64_t off = m * p.ldc + j;
        // optional outputs (uniform): no Z in the backward's recompute of G,
        // U; no G, U in the forward of the recompute mode
        if (Gp) store4(Gp + off, g[0], g[1], g[2], g[3]);
        if (Up) store4(Up + off, u[0], u[1], u[2], u[3]);
        if (Zp) store4(Zp + off, z[0], z[1], z[2], z[3]);
      }
    }
  } else {  // EPI_SWIGLU_BWD: acc = dZ; reload G, U; recompute the gate
    const T* Gp = static_cast<const T*>(p.g_in);
    const T* Up = static_cast<const T*>(p.u_in);
    T* dGp = static_cast<T*>(p.c0);
    T* dUp = static_cast<T*>(p.c1);
    T* Zp = static_cast<T*>(p.c2);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t m = m0 + wm * 128 + a * 16 + lrow;
      if (m >= p.M) continue;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t j = n0 + wn * 128 + b * 16 + lcol;
        if (j >= p.N) continue;
        const int64_t off = m * p.ldc + j;
        float g[4], u[4], dg[4], du[4], z[4];
        load4(Gp + off, g[0], g[1], g[2], g[3]);
        load4(Up + off, u[0], u[1], u[2], u[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sg = sigmoidf_fast(g[i]);
          const float act = g[i] * sg;
          const float dz = acc[a][b][i];
          dg[i] = dz * u[i] * sg * (1.0f + g[i] * (1.0f - sg));
          du[i] = dz * act;
          z[i] = act * u[i];
        }
        store4(dGp + off, dg[0], dg[1], dg[2], dg[3]);
        store4(dUp + off, du[0], du[1], du[2], du[3]);
        if (Zp) store4(Zp + off, z[0], z[1], z[2], z[3]);
      }
    }
  }
}

}  // namespace lmlp
