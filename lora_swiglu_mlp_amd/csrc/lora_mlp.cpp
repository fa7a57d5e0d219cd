// C ABI of the fused LoRA SwiGLU MLP: argument checks, buffer layout and the
// launch sequence. See include/lora_mlp.h for the contract.
//
// Forward (all on the caller's stream, no host synchronisation):
//   pack     adapter factors -> zero-padded operand layouts (those the backward
//            uses too go to `saved`)
//   rowproj  P_gu = X [A_g; A_u]^T            (fp32 -> saved; s*P_gu -> GEMM operand)
//   gemm     [G|U] = [X | sP_gu] [W|B]^T, epilogue G, U -> saved, Z = SiLU(G) U
//   rowproj  Pd = Z A_d^T                     (fp32 -> saved; s*Pd -> GEMM operand)
//   gemm     Y = [Z | sPd] [W_d | B_d]^T
// Backward:
//   rowproj  Q_d = dY B_d
//   gemm     dZ = [dY | sQ_d] [W_d ; A_d], epilogue: reload G, U, recompute
//            sigmoid(G), SiLU(G), Z; dG = dZ U sig (1 + G (1 - sig)), dU = dZ SiLU(G);
//            at rank <= 16 also the partials of Q_g = dG B_g, Q_u = dU B_u and of
//            dG^T P_g, dU^T P_u, Z^T Q_d (the last dZ tile columns may run as a
//            second launch of 128-wide tiles)
//   rowproj  Q_g = dG B_g, Q_u = dU B_u (rank > 16)
//   gemm     dX = [dG | dU | sQ_g | sQ_u] [W_g ; W_u ; A_g ; A_u]
//   colproj  X^T Q_gu, dY^T Pd (rank > 16 also dG^T P_g, dU^T P_u, Z^T Q_d), per token block
//   reduce   fixed-order sums, times s -> dB_g, dB_u, dA_d, dA_g, dA_u, dB_d
// This is the hand-derived backward of the fused LoRA MLP ("Unsloth 深度分析报告",
// section 创新之处) with the gate activations recomputed rather than stored
// (the "no materialised activations" point of the agientry.com unsloth page,
// section 训练侧).
#include "../../include/lora_mlp.h"

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "kernels.h"

namespace {

using namespace lmlp;

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

struct Dims {
  int64_t T, H, I, r, r16;
  float s;
  bool bf16, int4, consume;
  bool recompute;    // G, U not saved: the backward recomputes them
  bool q4_inkernel;  // 4-bit codes decoded inside the GEMM staging (else into bf16 copies)
  bool norm;         // RMSNorm in front of the MLP (the norm entry points)
  int eb;  // element bytes
  // tokens that size the row projections' K split (0: T). An expert of the
  // grouped MLP plans with the whole call's rows: its row projections run
  // merged with every other expert's, which fill the GPU together.
  int64_t t_split = 0;
};

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int parse_dims(const lmlp_dims* d, Dims& o) {
  if (!d) return fail(LMLP_ERR_INVALID_ARG, "dims is NULL");
  if (d->tokens < 0) return fail(LMLP_ERR_INVALID_ARG, "tokens < 0");
  if (d->hidden < 1 || d->inter < 1) return fail(LMLP_ERR_INVALID_ARG, "hidden and inter must be >= 1");
  if (d->rank < 1) return fail(LMLP_ERR_INVALID_ARG, "rank must be >= 1");
  if (!std::isfinite(d->scale)) return fail(LMLP_ERR_INVALID_ARG, "scale is not finite");
  if (d->dtype != LMLP_F32 && d->dtype != LMLP_BF16) return fail(LMLP_ERR_INVALID_ARG, "unknown dtype");
  if (d->wfmt != LMLP_W_DENSE && d->wfmt != LMLP_W_INT4_B64) return fail(LMLP_ERR_INVALID_ARG, "unknown wfmt");
  if (d->flags & ~(LMLP_CONSUME_SAVED | LMLP_INT4_INKERNEL | LMLP_RECOMPUTE_GU | LMLP_RMSNORM |
                   LMLP_INT4_BF16_COPIES))
    return fail(LMLP_ERR_INVALID_ARG, "unknown flag bits");
  if ((d->flags & LMLP_INT4_INKERNEL) && (d->flags & LMLP_INT4_BF16_COPIES))
    return fail(LMLP_ERR_INVALID_ARG, "LMLP_INT4_INKERNEL and LMLP_INT4_BF16_COPIES together");
  if (d->rank > 256) return fail(LMLP_ERR_UNSUPPORTED, "rank > 256");
  const int ch = d->dtype == LMLP_BF16 ? 8 : 4;
  if (d->hidden % ch || d->inter % ch)
    return fail(LMLP_ERR_UNSUPPORTED, "hidden and inter must be multiples of 8 (bf16) or 4 (fp32)");
  if (d->wfmt == LMLP_W_INT4_B64) {
    if (d->dtype != LMLP_BF16) return fail(LMLP_ERR_UNSUPPORTED, "4-bit weights need dtype bf16");
    if (d->hidden % 64 || d->inter % 64)
      return fail(LMLP_ERR_UNSUPPORTED, "4-bit weights need hidden and inter multiples of 64");
  }
  // sizes far beyond any one GPU; the DMA kernels address a 256-row operand
  // panel, or 128 token-contiguous bf16 rows of roundup(tokens, 64) elements,
  // with 32-bit buffer offsets and sizes: 128 * 2 * (2^24 - 64) < 2^32
  if (d->tokens > (int64_t{1} << 24) - 64 || d->hidden > (int64_t{1} << 22) || d->inter > (int64_t{1} << 22))
    return fail(LMLP_ERR_UNSUPPORTED, "dimension too large (tokens <= 2^24 - 64, hidden and inter <= 2^22)");
  o.T = d->tokens;
  o.H = d->hidden;
  o.I = d->inter;
  o.r = d->rank;
  o.r16 = (d->rank + 15) / 16 * 16;
  o.s = d->scale;
  o.bf16 = d->dtype == LMLP_BF16;
  o.int4 = d->wfmt == LMLP_W_INT4_B64;
  o.recompute = (d->flags & LMLP_RECOMPUTE_GU) != 0;
  o.consume = !o.recompute && (d->flags & LMLP_CONSUME_SAVED) != 0;
  o.q4_inkernel = o.int4 && (d->flags & LMLP_INT4_BF16_COPIES) == 0;
  o.norm = (d->flags & LMLP_RMSNORM) != 0;
  o.eb = o.bf16 ? 2 : 4;
  return LMLP_OK;
}

// The linear takes the MLP's dims (hidden = in, inter = out); of the flags
// only LMLP_INT4_INKERNEL and LMLP_INT4_BF16_COPIES apply to it.
int parse_linear_dims(const lmlp_dims* d, Dims& o) {
  if (d && (d->flags & ~(LMLP_INT4_INKERNEL | LMLP_INT4_BF16_COPIES)))
    return fail(LMLP_ERR_INVALID_ARG, "flags other than INT4_INKERNEL, INT4_BF16_COPIES");
  return parse_dims(d, o);
}

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  }
};

// The adapter factors in the operand layouts both passes use are packed once,
// by the forward, next to the activations (the backward gets the same
// weights).
struct SavedLayout {
  size_t g, u, pgu, pd, agu_pad, ad_pad, bdT, bgT, buT, bext_g, bext_u, rstd, total;
};
SavedLayout saved_layout(const Dims& d) {
  Carver c;
  SavedLayout L;
  L.g = d.recompute ? 0 : c.take(size_t(d.T) * d.I * d.eb);
  L.u = d.recompute ? 0 : c.take(size_t(d.T) * d.I * d.eb);
  L.pgu = c.take(size_t(d.T) * 2 * d.r16 * 4);
  L.pd = c.take(size_t(d.T) * d.r16 * 4);
  L.agu_pad = c.take(size_t(2 * d.r16) * d.H * d.eb);  // [A_g; A_u], rank rows zero-padded
  L.ad_pad = c.take(size_t(d.r16) * d.I * d.eb);       // A_d
  L.bdT = c.take(size_t(d.r16) * d.H * d.eb);          // B_d^T
  L.bgT = c.take(size_t(d.r16) * d.I * d.eb);          // B_g^T
  L.buT = c.take(size_t(d.r16) * d.I * d.eb);          // B_u^T
  // B_g, B_u as [I, 2 r16] (rank along K, padded): the gate/up product's
  // adapter segment, which the backward reruns with LMLP_RECOMPUTE_GU
  L.bext_g = c.take(size_t(d.I) * 2 * d.r16 * d.eb);
  L.bext_u = c.take(size_t(d.I) * 2 * d.r16 * d.eb);
  L.rstd = d.norm ? c.take(size_t(d.T) * 4) : 0;  // the norm's statistics, reused by the backward
  L.total = c.off;
  return L;
}

// Split-K plan of a row projection over a [T, K] activation with n1p output
// columns. bf16 (LDS-streamed kernel, 128-row workgroups of up to 32 or 64
// columns, two per CU): about 256 workgroups (measured a little faster than
// 512), slices in whole 64-element stages. fp32: about 768 workgroups of 256
// rows, at least 256 elements per slice.
struct RpPlan {
  int ks;
  int64_t kb;
};
RpPlan rp_plan(const Dims& d, int64_t K, int n1p) {
  const int64_t Ts = d.t_split > 0 ? d.t_split : d.T;
  if (d.bf16) {
    const int64_t work = std::max<int64_t>(1, (Ts + 127) / 128 * (n1p > 32 ? (n1p + 63) / 64 : 1));
    int64_t ks = (256 + work - 1) / work;
    ks = std::min(std::max<int64_t>(ks, 1), std::max<int64_t>(1, K / 128));
    int64_t kb = (K + ks - 1) / ks;
    kb = (kb + 63) / 64 * 64;
    return {static_cast<int>((K + kb - 1) / kb), kb};
  }
  const int64_t unit = 4 * 16;  // one load batch: four MFMA k-steps
  const int64_t work = std::max<int64_t>(1, (Ts + 255) / 256 * ((n1p + 63) / 64));
  int64_t ks = (768 + work - 1) / work;
  ks = std::min(std::max<int64_t>(ks, 1), std::max<int64_t>(1, K / 256));
  int64_t kb = (K + ks - 1) / ks;
  kb = (kb + unit - 1) / unit * unit;
  return {static_cast<int>((K + kb - 1) / kb), kb};
}
size_t rp_part_bytes(const Dims& d, int64_t K, int n1p) {
  return size_t(rp_plan(d, K, n1p).ks) * size_t(d.T) * size_t(n1p) * 4;
}

// bf16 with r <= 16: the dZ GEMM's epilogue also forms the row projections
// dG B_g and dU B_u (one split-K slice per 256-column tile of I) and the
// column products P_g^T dG, P_u^T dU and Q_d^T Z (one slice per 256-row tile).
// The fused epilogue addresses a 256-row tile of G and U with 32-bit byte
// offsets (256 * I * 2 bytes must stay below 2^31).
bool fused_q(const Dims& d) { return d.bf16 && d.r16 == 16 && d.I < (int64_t(1) << 22); }
// Row-product slices at most (every column in 128-wide tiles); the actual
// count follows the dZ GEMM's split (dz_split).
int64_t q_slices(const Dims& d) { return (d.I + 127) / 128; }
int64_t col_slices(const Dims& d) { return (d.T + 255) / 256; }
size_t q_part_bytes(const Dims& d) {
  return fused_q(d) ? size_t(q_slices(d)) * size_t(d.T) * size_t(d.r16) * 4 : 0;
}

// Compute units of the current device.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

// Tile width of a bf16 product with the plain store epilogue: 256 x 128 tiles
// when 256 x 256 ones would not fill one wave of the device (narrow outputs,
// few tokens), else the default 256 x 256.
int store_tile_n(const Dims& d, int64_t M, int64_t N) {
  if (!d.bf16) return 0;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return tiles < device_cus() ? 128 : 0;
}

// K splits of the linear's bf16 forward product when its 256 x 256 tiles
// would fill less than one wave of the device: each split runs every tile
// over a slice of K and stores fp32 partials, which a sum kernel adds in
// split order. At most 8 splits, each over at least 512 of K, partials of at
// most 64 MiB, N a multiple of 4. Dense weights only. 1 = no split.
int linear_splitk(const Dims& d) {
  if (!d.bf16 || d.int4 || d.T == 0 || d.I % 4) return 1;
  const int64_t tiles = ((d.T + 255) / 256) * ((d.I + 255) / 256);
  const int64_t ncu = device_cus();
  if (tiles >= ncu) return 1;
  int64_t s = (ncu + tiles - 1) / tiles;
  s = std::min<int64_t>(s, 8);
  s = std::min<int64_t>(s, d.H / 512);
  while (s > 1 && s * d.T * d.I * 4 > (int64_t(64) << 20)) --s;
  return s > 1 ? static_cast<int>(s) : 1;
}

// Columns of the dZ GEMM (bf16) covered by 256-wide tiles; the rest, when the
// last wave of workgroups would be at most half full, goes to a second launch
// of 128-wide tiles that fill one wave with twice as many half-size tiles.
int64_t dz_split(const Dims& d) {
  if (!d.bf16) return d.I;
  const int64_t ncu = device_cus();
  const int64_t tm = (d.T + 255) / 256, tn = (d.I + 255) / 256;
  const int64_t tiles = tm * tn, rem = tiles % ncu;
  if (tiles <= ncu || rem == 0 || 2 * rem > ncu) return d.I;
  const int64_t ntail = (rem + tm - 1) / tm;  // 256-wide tile columns moved to the tail
  if (ntail >= tn || tm * ntail * 2 > ncu) return d.I;
  return (tn - ntail) * 256;
}

// token blocks of the column projections (partial sums over tokens). bf16:
// at most 8; more blocks measured slower at 8K and 32K tokens (more partials
// to write and reduce, no gain in streaming rate).
int colproj_ntb(const Dims& d) {
  if (d.T <= 0) return 0;
  if (d.bf16) return static_cast<int>(std::min<int64_t>(8, std::max<int64_t>(1, (d.T + 511) / 512)));
  return static_cast<int>(std::min<int64_t>(16, (d.T + 255) / 256));
}
int64_t colproj_tr(int64_t T, int ntb) {
  if (ntb == 0) return 32;
  const int64_t per = (T + ntb - 1) / ntb;
  return (per + 31) / 32 * 32;
}
int64_t ld_tok(const Dims& d) { return (d.T + 63) / 64 * 64; }  // token-contiguous rows

// fp32 scales per row of a 4-bit weight in the NN products' layout: the
// in/64 blocks padded to a multiple of 4 (16-byte rows)
int64_t sc_ld4(int64_t in) { return (in / 64 + 3) / 4 * 4; }

struct FwdLayout {
  size_t z, aext_gu, aext_d, bext_d, rp_part, sc_g, sc_u, sc_d;
  size_t wq_g, wq_u, wq_d, xn, total;
};
FwdLayout fwd_layout(const Dims& d) {
  Carver c;
  FwdLayout L;
  L.z = c.take(size_t(d.T) * d.I * d.eb);
  L.aext_gu = c.take(size_t(d.T) * 2 * d.r16 * d.eb);
  L.aext_d = c.take(size_t(d.T) * d.r16 * d.eb);
  L.bext_d = c.take(size_t(d.H) * d.r16 * d.eb);
  L.rp_part = c.take(std::max(rp_part_bytes(d, d.H, int(2 * d.r16)), rp_part_bytes(d, d.I, int(d.r16))));
  // 4-bit weights decoded in the GEMMs: block scales as fp32, block-major
  // ([in/64][out]); otherwise bf16 copies of the weights
  const bool ink = d.q4_inkernel, cp = d.int4 && !d.q4_inkernel;
  L.sc_g = ink ? c.take(size_t(d.H / 64) * d.I * 4 + 16) : 0;
  L.sc_u = ink ? c.take(size_t(d.H / 64) * d.I * 4 + 16) : 0;
  L.sc_d = ink ? c.take(size_t(d.I / 64) * d.H * 4 + 16) : 0;
  L.wq_g = cp ? c.take(size_t(d.I) * d.H * 2) : 0;
  L.wq_u = cp ? c.take(size_t(d.I) * d.H * 2) : 0;
  L.wq_d = cp ? c.take(size_t(d.H) * d.I * 2) : 0;
  L.xn = d.norm ? c.take(size_t(d.T) * d.H * d.eb) : 0;  // the normalised rows
  L.total = c.off;
  return L;
}

struct BwdLayout {
  size_t g_rc, u_rc, dg, du, z, qd, aext_d, qgu, aext_gu;
  size_t rp_a, rp_b, pguT, pdT, qdT, qguT, wq_g, wq_u, wq_d, scn_g, scn_u, scn_d, sct_g, sct_u;
  size_t part_dg, part_du, part_z, part_x, part_dy, xn, total;
  int ntb;
  int64_t tr;
};
BwdLayout bwd_layout(const Dims& d) {
  Carver c;
  BwdLayout L;
  L.ntb = colproj_ntb(d);
  L.tr = colproj_tr(d.T, L.ntb);
  const size_t act = size_t(d.T) * d.I * d.eb;
  // LMLP_RECOMPUTE_GU: G, U recomputed here; dG, dU overwrite them
  L.g_rc = d.recompute ? c.take(act) : 0;
  L.u_rc = d.recompute ? c.take(act) : 0;
  L.dg = d.consume || d.recompute ? 0 : c.take(act);
  L.du = d.consume || d.recompute ? 0 : c.take(act);
  L.z = c.take(act);
  L.qd = c.take(size_t(d.T) * d.r16 * 4);
  L.aext_d = c.take(size_t(d.T) * d.r16 * d.eb);
  L.qgu = c.take(size_t(d.T) * 2 * d.r16 * 4);
  L.aext_gu = c.take(size_t(d.T) * 2 * d.r16 * d.eb);
  L.rp_a = c.take(std::max({rp_part_bytes(d, d.H, int(d.r16)), rp_part_bytes(d, d.I, int(d.r16)), q_part_bytes(d)}));
  L.rp_b = c.take(std::max(rp_part_bytes(d, d.I, int(d.r16)), q_part_bytes(d)));
  // transposed, token-contiguous copies of the [T, r] operands of the column
  // projections (bf16 path only)
  const size_t trow = d.bf16 ? size_t(ld_tok(d)) * d.eb : 0;
  L.pguT = c.take(2 * d.r16 * trow);
  L.pdT = c.take(d.r16 * trow);
  L.qdT = c.take(d.r16 * trow);
  L.qguT = c.take(2 * d.r16 * trow);
  // 4-bit weights: bf16 copies for the products (decoded once per call), or
  // with the decode in the GEMM staging the fp32 block scales: row-major with
  // rows padded to 4 blocks for the NN products, block-major for the gate/up
  // product the recompute mode reruns
  const bool cp = d.int4 && !d.q4_inkernel, ink = d.q4_inkernel;
  L.wq_g = cp ? c.take(size_t(d.I) * d.H * 2) : 0;
  L.wq_u = cp ? c.take(size_t(d.I) * d.H * 2) : 0;
  L.wq_d = cp ? c.take(size_t(d.H) * d.I * 2) : 0;
  L.scn_g = ink ? c.take(size_t(d.I) * sc_ld4(d.H) * 4 + 16) : 0;
  L.scn_u = ink ? c.take(size_t(d.I) * sc_ld4(d.H) * 4 + 16) : 0;
  L.scn_d = ink ? c.take(size_t(d.H) * sc_ld4(d.I) * 4 + 16) : 0;
  L.sct_g = ink && d.recompute ? c.take(size_t(d.H / 64) * d.I * 4 + 16) : 0;
  L.sct_u = ink && d.recompute ? c.take(size_t(d.H / 64) * d.I * 4 + 16) : 0;
  const size_t nsl_i = fused_q(d) ? size_t(col_slices(d)) : size_t(L.ntb);
  L.part_dg = c.take(nsl_i * d.I * d.r16 * 4);
  L.part_du = c.take(nsl_i * d.I * d.r16 * 4);
  L.part_z = c.take(nsl_i * d.I * d.r16 * 4);
  L.part_x = c.take(size_t(L.ntb) * d.H * 2 * d.r16 * 4);
  L.part_dy = c.take(size_t(L.ntb) * d.H * d.r16 * 4);
  L.xn = d.norm ? c.take(size_t(d.T) * d.H * d.eb) : 0;  // the normalised rows, re-applied
  L.total = c.off;
  return L;
}

// ---- fused LoRA linear: y = x W^T + s (x A^T) B^T, in = H, out = I of Dims
struct LinSavedLayout {
  size_t p, pT, a_pad, bext, bT, total;
};
LinSavedLayout lin_saved_layout(const Dims& d) {
  Carver c;
  LinSavedLayout L;
  L.p = c.take(size_t(d.T) * d.r16 * 4);                                // x A^T fp32
  L.pT = d.bf16 ? c.take(size_t(d.r16) * ld_tok(d) * d.eb) : 0;        // its transposed copy
  L.a_pad = c.take(size_t(d.r16) * d.H * d.eb);                         // A, rank rows padded
  L.bext = c.take(size_t(d.I) * d.r16 * d.eb);                          // B as [out, r16]
  L.bT = c.take(size_t(d.r16) * d.I * d.eb);                            // B^T as [r16, out]
  L.total = c.off;
  return L;
}
struct LinFwdLayout {
  size_t aext, rp_part, sc, wq, ypart, total;
  int nsplit;
};
LinFwdLayout lin_fwd_layout(const Dims& d) {
  Carver c;
  LinFwdLayout L;
  L.aext = c.take(size_t(d.T) * d.r16 * d.eb);  // s x A^T, the product's adapter segment
  L.rp_part = c.take(rp_part_bytes(d, d.H, int(d.r16)));
  L.sc = d.q4_inkernel ? c.take(size_t(d.H / 64) * d.I * 4 + 16) : 0;
  L.wq = d.int4 && !d.q4_inkernel ? c.take(size_t(d.I) * d.H * 2) : 0;
  L.nsplit = linear_splitk(d);
  L.ypart = L.nsplit > 1 ? c.take(size_t(L.nsplit) * d.T * d.I * 4) : 0;  // fp32 split-K partials of y
  L.total = c.off;
  return L;
}
struct LinBwdLayout {
  size_t q, aext, qT, rp_part, part_x, part_dy, wq, scn, total;
  int ntb;
  int64_t tr;
};
LinBwdLayout lin_bwd_layout(const Dims& d) {
  Carver c;
  LinBwdLayout L;
  L.ntb = colproj_ntb(d);
  L.tr = colproj_tr(d.T, L.ntb);
  L.q = c.take(size_t(d.T) * d.r16 * 4);                          // dy B fp32
  L.aext = c.take(size_t(d.T) * d.r16 * d.eb);                    // s dy B, the dX product's segment
  L.qT = d.bf16 ? c.take(size_t(d.r16) * ld_tok(d) * d.eb) : 0;  // its transposed copy
  L.rp_part = c.take(rp_part_bytes(d, d.I, int(d.r16)));
  L.part_x = c.take(size_t(L.ntb) * d.H * d.r16 * 4);
  L.part_dy = c.take(size_t(L.ntb) * d.I * d.r16 * 4);
  // 4-bit W: a bf16 copy for the NN product, or (decoded in the staging) its
  // fp32 scales, row-major with rows padded to 4 blocks
  L.wq = d.int4 && !d.q4_inkernel ? c.take(size_t(d.I) * d.H * 2) : 0;
  L.scn = d.q4_inkernel ? c.take(size_t(d.I) * sc_ld4(d.H) * 4 + 16) : 0;
  L.total = c.off;
  return L;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int need_ptr(const void* p, const char* name) {
  if (!p) return fail(LMLP_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p)) return fail(LMLP_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return LMLP_OK;
}

#define LMLP_TRY(expr)            \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != LMLP_OK) return rc_; \
  } while (0)

int check_weights(const Dims& d, const void* wg, const void* wgs, const void* wu, const void* wus,
                  const void* wd, const void* wds) {
  LMLP_TRY(need_ptr(wg, "w_gate"));
  LMLP_TRY(need_ptr(wu, "w_up"));
  LMLP_TRY(need_ptr(wd, "w_down"));
  if (d.int4) {
    LMLP_TRY(need_ptr(wgs, "w_gate_scales"));
    LMLP_TRY(need_ptr(wus, "w_up_scales"));
    LMLP_TRY(need_ptr(wds, "w_down_scales"));
  } else if (wgs || wus || wds) {
    return fail(LMLP_ERR_INVALID_ARG, "scale pointers must be NULL for dense weights");
  }
  return LMLP_OK;
}

int check_adapters(const void* ag, const void* bg, const void* au, const void* bu, const void* ad,
                   const void* bd) {
  LMLP_TRY(need_ptr(ag, "a_gate"));
  LMLP_TRY(need_ptr(bg, "b_gate"));
  LMLP_TRY(need_ptr(au, "a_up"));
  LMLP_TRY(need_ptr(bu, "b_up"));
  LMLP_TRY(need_ptr(ad, "a_down"));
  LMLP_TRY(need_ptr(bd, "b_down"));
  return LMLP_OK;
}

// gfx950 check, cached per device
int check_device() {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LMLP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(LMLP_ERR_UNSUPPORTED, "device index out of range");
  int st = cache[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(LMLP_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(LMLP_ERR_UNSUPPORTED, "current device is not gfx950");
  return LMLP_OK;
}

int hip_rc(hipError_t e, const char* what) {
  if (e == hipSuccess) return LMLP_OK;
  return fail(LMLP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---- optional per-launch timing (lora_mlp_profile_begin / _end)
struct ProfRec {
  const char* name;
  hipEvent_t b, e;
};
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<ProfRec> recs;
  hipEvent_t next() {
    if (used == pool.size()) {
      hipEvent_t ev = nullptr;
      if (hipEventCreate(&ev) != hipSuccess) return nullptr;
      pool.push_back(ev);
    }
    return pool[used++];
  }
};
thread_local Profiler g_prof;
constexpr size_t kMaxProfiled = 65536;

struct ProfScope {
  hipStream_t st;
  const char* name;
  hipEvent_t b = nullptr;
  ProfScope(hipStream_t s, const char* n) : st(s), name(n) {
    if (g_prof.on && g_prof.recs.size() < kMaxProfiled) {
      b = g_prof.next();
      if (b) hipEventRecord(b, st);
    }
  }
  void done() {
    if (!b) return;
    hipEvent_t e = g_prof.next();
    if (!e) return;
    hipEventRecord(e, st);
    g_prof.recs.push_back({name, b, e});
  }
};

#define LMLP_LAUNCH(name, expr)                  \
  do {                                           \
    ProfScope ps_(st, name);                     \
    LMLP_TRY(hip_rc((expr), name));              \
    ps_.done();                                  \
  } while (0)

// Phase control of one forward or backward pass, for the grouped MLP: the
// pass is cut at its GEMMs. phase < 0: everything runs (the plain entry
// points). phase k: only the side kernels between GEMM k-1 and GEMM k are
// launched, and GEMM k is handed back in `gp` instead of being launched (the
// pass returns there); a pass with no GEMM left hands back nothing. Running
// phases 0, 1, ... in order launches the same work in the same order.
struct Exec {
  int64_t t_split = 0;  // Dims::t_split of the pass (grouped MLP)
  int phase = -1;
  int seg = 0;  // GEMMs passed so far
  bool sunk = false;
  const char* name = nullptr;
  GemmParams gp{};
  int nn = 0, epi = 0;
  bool groupable = false;  // a dense bf16 product (the grouped launcher takes it)
  std::vector<struct SideOp>* rec = nullptr;  // record the batchable side kernels here instead of launching
  bool side() const { return phase < 0 || seg == phase; }
};

// A recorded side-kernel launch of a grouped pass: its kind, flag (element
// bytes for pack, bf16 for the others) and jobs (each with its own token
// count), to be launched merged with the same launch of the other experts.
enum SideKind { SK_PACK = 0, SK_ROWPROJ, SK_FINISH, SK_COLPROJ, SK_REDUCE };
struct SideOp {
  const char* name;
  int kind, flag;
  std::vector<char> jobs;  // njobs jobs of the kind's job type
  int njobs;
};
template <typename J>
SideOp side_op_of(const char* name, int kind, int flag, const J* jobs, int n, int64_t T) {
  SideOp o{name, kind, flag, {}, n};
  std::vector<J> js(jobs, jobs + n);
  if constexpr (!std::is_same<J, PackJob>::value && !std::is_same<J, ReduceJob>::value)
    for (J& j : js)
      if (j.T == 0) j.T = T;
  (void)T;
  o.jobs.assign(reinterpret_cast<const char*>(js.data()), reinterpret_cast<const char*>(js.data() + n));
  return o;
}
SideOp side_op(const char* n, int kind, const PackParams& p, int flag) {
  return side_op_of(n, kind, flag, p.job, p.njobs, 0);
}
SideOp side_op(const char* n, int kind, const RowProjParams& p, int flag) {
  return side_op_of(n, kind, flag, p.job, p.njobs, p.T);
}
SideOp side_op(const char* n, int kind, const ProjFinishParams& p, int flag) {
  return side_op_of(n, kind, flag, p.job, p.njobs, p.T);
}
SideOp side_op(const char* n, int kind, const ColProjParams& p, int flag) {
  return side_op_of(n, kind, flag, p.job, p.njobs, p.T);
}
SideOp side_op(const char* n, int kind, const ReduceParams& p, int flag) {
  return side_op_of(n, kind, flag, p.job, p.njobs, 0);
}

// Device job tables of the merged side launches: room per expert for the
// most jobs one of its side launches carries (the forward's packing, 10).
constexpr size_t kSideJobBytes = 96;
constexpr size_t kSideJobsPerExpert = 10;
static_assert(sizeof(PackJob) <= kSideJobBytes && sizeof(RowProjJob) <= kSideJobBytes &&
                  sizeof(ProjFinishJob) <= kSideJobBytes && sizeof(ColProjJob) <= kSideJobBytes &&
                  sizeof(ReduceJob) <= kSideJobBytes,
              "side job table entries");

// One kind's recorded jobs: with a job table batch, one launch (at most 8190
// jobs each) reading its jobs from the table, deferred to the batch; else
// merged into launches of up to the job capacity of the kernel arguments
// (deferred to the batch too when there is one, so that the order holds).
template <typename P, typename L>
hipError_t launch_jobs(const std::vector<const SideOp*>& ops, bool has_t, TableBatch* tb, L launch) {
  using J = typename std::remove_reference<decltype(P{}.job[0])>::type;
  constexpr int cap = int(sizeof(P{}.job) / sizeof(J));
  size_t total = 0;
  for (const SideOp* o : ops) total += size_t(o->njobs);
  if (tb && total > size_t(cap)) {
    auto all = std::make_shared<std::vector<J>>();
    all->reserve(total);
    P q{};
    for (const SideOp* o : ops) {
      const J* js = reinterpret_cast<const J*>(o->jobs.data());
      for (int i = 0; i < o->njobs; ++i) {
        all->push_back(js[i]);
        if constexpr (!std::is_same<J, PackJob>::value && !std::is_same<J, ReduceJob>::value)
          if (has_t && js[i].T > q.T) q.T = js[i].T;
      }
    }
    void* dtab = tb->add(all->data(), total * sizeof(J));
    if (!dtab) {
      const hipError_t e = tb->make_room();
      if (e != hipSuccess) return e;
      dtab = tb->add(all->data(), total * sizeof(J));
      if (!dtab) return hipErrorInvalidValue;  // larger than the whole batch
    }
    // at most 8190 jobs per launch: the job index rides in a grid dimension
    // (65535), times up to 8 column slices for the row projections
    constexpr size_t kMaxJobs = 8190;
    for (size_t j0 = 0; j0 < total; j0 += kMaxJobs) {
      P qj = q;
      qj.njobs = static_cast<int32_t>(std::min(kMaxJobs, total - j0));
      qj.table = static_cast<const J*>(dtab) + j0;
      tb->defer([qj, all, j0, launch]() { return launch(qj, all->data() + j0); });
    }
    return hipSuccess;
  }
  P q{};
  auto flush = [&]() -> hipError_t {
    if (q.njobs == 0) return hipSuccess;
    hipError_t e = hipSuccess;
    if (tb) {
      const P qq = q;
      tb->defer([qq, launch]() { return launch(qq, nullptr); });
    } else {
      e = launch(q, nullptr);
    }
    q = P{};
    return e;
  };
  for (const SideOp* o : ops) {
    const J* js = reinterpret_cast<const J*>(o->jobs.data());
    for (int i = 0; i < o->njobs; ++i) {
      q.job[q.njobs++] = js[i];
      if constexpr (!std::is_same<J, PackJob>::value && !std::is_same<J, ReduceJob>::value)
        if (has_t && js[i].T > q.T) q.T = js[i].T;
      if (q.njobs == cap) {
        const hipError_t e = flush();
        if (e != hipSuccess) return e;
      }
    }
  }
  return flush();
}

hipError_t launch_side_group(const std::vector<const SideOp*>& ops, hipStream_t st, TableBatch* tb) {
  const int kind = ops[0]->kind, flag = ops[0]->flag;
  switch (kind) {
    case SK_PACK:
      return launch_jobs<PackParams>(ops, false, tb, [flag, st](const PackParams& q, const PackJob* h) {
        return launch_pack(q, flag, st, h);
      });
    case SK_ROWPROJ:
      return launch_jobs<RowProjParams>(ops, true, tb, [flag, st](const RowProjParams& q, const RowProjJob* h) {
        return launch_rowproj(q, flag, st, h);
      });
    case SK_FINISH:
      return launch_jobs<ProjFinishParams>(ops, true, tb,
                                           [flag, st](const ProjFinishParams& q, const ProjFinishJob* h) {
                                             return launch_proj_finish(q, flag, st, h);
                                           });
    case SK_COLPROJ:
      return launch_jobs<ColProjParams>(ops, true, tb, [flag, st](const ColProjParams& q, const ColProjJob* h) {
        return launch_colproj(q, flag, st, h);
      });
    case SK_REDUCE:
      return launch_jobs<ReduceParams>(ops, false, tb, [st](const ReduceParams& q, const ReduceJob* h) {
        return launch_reduce(q, st, h);
      });
    default:
      return hipErrorInvalidValue;
  }
}

#define LMLP_SIDE_REC(name, kind, params, flag, launch_expr)                   \
  do {                                                                          \
    if (ex.side()) {                                                            \
      if (ex.rec) ex.rec->push_back(side_op(name, kind, params, flag));         \
      else LMLP_LAUNCH(name, launch_expr);                                      \
    }                                                                           \
  } while (0)

#define LMLP_SIDE(name, expr)                  \
  do {                                         \
    if (ex.side()) LMLP_LAUNCH(name, expr);    \
  } while (0)

#define LMLP_GEMM(name_, gp_, nn_, epi_)                                          \
  do {                                                                             \
    if (ex.phase < 0) {                                                            \
      LMLP_LAUNCH(name_, run_gemm(gp_, d, nn_, epi_, st));                         \
    } else if (ex.seg == ex.phase) {                                               \
      ex.sunk = true;                                                              \
      ex.name = name_;                                                             \
      ex.gp = gp_;                                                                 \
      ex.nn = nn_;                                                                 \
      ex.epi = epi_;                                                               \
      ex.groupable = d.bf16 && !(gp_).seg[0].bint4;                                \
      return LMLP_OK;                                                              \
    }                                                                              \
    ++ex.seg;                                                                      \
  } while (0)

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

// bf16 products take the LDS-DMA kernels (4-bit weights decoded in the
// staging: the decoding variant); fp32 products the general kernel.
// products with 4-bit B segments: the eight-wave decoding kernel, 256-wide tiles
hipError_t run_q4(const GemmParams& p, int nn, int epi, hipStream_t st) {
  GemmParams q = p;
  q.tile_n = 0;
  return launch_gemm_bf16_q4(q, nn, epi, st);
}

hipError_t run_gemm(const GemmParams& p, const Dims& d, int nn, int epi, hipStream_t st) {
  if (!d.bf16) return launch_gemm_f32(p, nn, epi, st);
  if (p.seg[0].bint4) return run_q4(p, nn, epi, st);
  return launch_gemm_bf16(p, nn, epi, st);
}

PackJob pack_job(void* dst, int64_t ld_dst, int64_t rows, int64_t cols, const void* src, int64_t ld_src,
                 int64_t srows, int64_t scols, bool transpose) {
  PackJob j{};
  j.dst = dst;
  j.ld_dst = ld_dst;
  j.rows = rows;
  j.cols = cols;
  j.src = src;
  j.ld_src = ld_src;
  j.srows = srows;
  j.scols = scols;
  j.transpose = transpose ? 1 : 0;
  return j;
}

GemmSeg seg(const void* a, int64_t lda, const void* b0, const void* b1, int64_t ldb, int64_t K,
            bool bint4 = false, const void* bs0 = nullptr, const void* bs1 = nullptr) {
  GemmSeg s{};
  s.a = a;
  s.lda = lda;
  s.b0 = b0;
  s.b1 = b1;
  s.ldb = ldb;
  s.K = K;
  s.bint4 = bint4 ? 1 : 0;
  s.bs0 = bs0;
  s.bs1 = bs1;
  return s;
}

RowProjJob rp_job(const Dims& d, const void* x, int64_t ldx, int64_t K, const void* w, int64_t ldw, int n1p,
                  float* part) {
  const RpPlan pl = rp_plan(d, K, n1p);
  RowProjJob j{};
  j.x = x;
  j.ldx = ldx;
  j.K = K;
  j.w = w;
  j.ldw = ldw;
  j.n1p = n1p;
  j.part = part;
  j.kb = pl.kb;
  j.kslices = pl.ks;
  return j;
}

ProjFinishJob fin_job(const float* part, int nparts, int64_t part_stride, int64_t ld_part, int n1p, float* out_f32,
                      int64_t ld_f32, void* out_c, int64_t ld_c, float scale, void* outT, int64_t ldT, int col_off) {
  ProjFinishJob j{};
  j.part = part;
  j.nparts = nparts;
  j.part_stride = part_stride;
  j.ld_part = ld_part;
  j.n1p = n1p;
  j.out_f32 = out_f32;
  j.ld_f32 = ld_f32;
  j.out_c = out_c;
  j.ld_c = ld_c;
  j.scale = scale;
  j.outT = outT;
  j.ldT = ldT;
  j.col_off = col_off;
  return j;
}

ColProjJob cp_job(const Dims& d, const void* x, int64_t ldx, int64_t K, const float* p, int64_t ldp, const void* pT,
                  int64_t ldpT, int n2p, float* part, int ntb, int64_t tr) {
  ColProjJob j{};
  j.x = x;
  j.ldx = ldx;
  j.K = K;
  j.p = p;
  j.ldp = ldp;
  j.pT = pT;
  j.ldpT = ldpT;
  j.n2p = n2p;
  j.part = part;
  j.ntb = ntb;
  j.tr = tr;
  j.kblocks = static_cast<int>(d.bf16 ? (K + 255) / 256 : (K + 63) / 64);
  j.nchunks = d.bf16 ? (n2p + 127) / 128 : (n2p + 63) / 64;
  return j;
}

ReduceJob rd_job(const float* src, int64_t chunk_stride, int nchunk, int64_t ld_src, int col_off, int64_t rows,
                 int64_t cols, void* dst, int64_t ld_dst, bool transpose, float scale, bool bf16) {
  ReduceJob j{};
  j.src = src;
  j.chunk_stride = chunk_stride;
  j.nchunk = nchunk;
  j.ld_src = ld_src;
  j.col_off = col_off;
  j.rows = rows;
  j.cols = cols;
  j.dst = dst;
  j.ld_dst = ld_dst;
  j.transpose = transpose ? 1 : 0;
  j.scale = scale;
  j.dst_bf16 = bf16 ? 1 : 0;
  return j;
}

}  // namespace

extern "C" {

size_t lora_mlp_saved_bytes(const lmlp_dims* dims) {
  Dims d;
  if (parse_dims(dims, d) != LMLP_OK) return 0;
  return saved_layout(d).total;
}

size_t lora_mlp_workspace_bytes(const lmlp_dims* dims, int is_backward) {
  Dims d;
  if (parse_dims(dims, d) != LMLP_OK) return 0;
  return is_backward ? bwd_layout(d).total : fwd_layout(d).total;
}

const char* lora_mlp_status_string(int status) {
  switch (status) {
    case LMLP_OK: return "LMLP_OK";
    case LMLP_ERR_INVALID_ARG: return "LMLP_ERR_INVALID_ARG";
    case LMLP_ERR_UNSUPPORTED: return "LMLP_ERR_UNSUPPORTED";
    case LMLP_ERR_WORKSPACE: return "LMLP_ERR_WORKSPACE";
    case LMLP_ERR_HIP: return "LMLP_ERR_HIP";
    default: return "LMLP_UNKNOWN_STATUS";
  }
}

const char* lora_mlp_last_error(void) { return g_last_error.c_str(); }

// The MLP forward; with dims.flags & LMLP_RMSNORM the rows of x are first
// normalised (gamma, eps) and the MLP runs on the result.
static int forward_impl(const lmlp_dims* dims, const void* gamma, float eps, const void* x, const void* w_gate,
                        const void* w_gate_scales, const void* w_up, const void* w_up_scales, const void* w_down,
                        const void* w_down_scales, const void* a_gate, const void* b_gate, const void* a_up,
                        const void* b_up, const void* a_down, const void* b_down, void* y, void* saved,
                        size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                        Exec* exec = nullptr) {
  Exec local_exec;
  Exec& ex = exec ? *exec : local_exec;
  Dims d;
  LMLP_TRY(parse_dims(dims, d));
  d.t_split = ex.t_split;
  if (d.norm) LMLP_TRY(need_ptr(gamma, "gamma"));
  LMLP_TRY(check_weights(d, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales));
  LMLP_TRY(check_adapters(a_gate, b_gate, a_up, b_up, a_down, b_down));
  const SavedLayout SL = saved_layout(d);
  const FwdLayout FL = fwd_layout(d);
  if (d.T > 0) {
    LMLP_TRY(need_ptr(x, "x"));
    LMLP_TRY(need_ptr(y, "y"));
    LMLP_TRY(need_ptr(saved, "saved"));
    LMLP_TRY(need_ptr(workspace, "workspace"));
  }
  if (saved_bytes < SL.total) return fail(LMLP_ERR_WORKSPACE, "saved buffer smaller than lora_mlp_saved_bytes()");
  if (workspace_bytes < FL.total)
    return fail(LMLP_ERR_WORKSPACE, "workspace smaller than lora_mlp_workspace_bytes(dims, 0)");
  LMLP_TRY(check_device());
  if (d.T == 0) return LMLP_OK;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t T = d.T, H = d.H, I = d.I, r = d.r, r16 = d.r16;
  if (d.norm) {  // xn = RMSNorm(x); rstd kept for the backward
    NormParams np{};
    np.x = x;
    np.gamma = gamma;
    np.xn = at(workspace, FL.xn);
    np.rstd = reinterpret_cast<float*>(at(saved, SL.rstd));
    np.T = T;
    np.H = H;
    np.eps = eps;
    np.mode = NORM_FWD;
    LMLP_SIDE("rmsnorm(fwd)", launch_rmsnorm(np, d.bf16, st));
    x = np.xn;
  }
  // with LMLP_RECOMPUTE_GU the gate/up epilogue stores only Z
  char* G = d.recompute ? nullptr : at(saved, SL.g);
  char* U = d.recompute ? nullptr : at(saved, SL.u);
  float* Pgu = reinterpret_cast<float*>(at(saved, SL.pgu));
  float* Pd = reinterpret_cast<float*>(at(saved, SL.pd));
  char* Z = at(workspace, FL.z);
  char* aext_gu = at(workspace, FL.aext_gu);
  char* aext_d = at(workspace, FL.aext_d);
  char* agu_pad = at(saved, SL.agu_pad);
  char* ad_pad = at(saved, SL.ad_pad);
  char* bext_g = at(saved, SL.bext_g);
  char* bext_u = at(saved, SL.bext_u);
  char* bext_d = at(workspace, FL.bext_d);
  const int eb = d.eb;

  PackParams pk{};
  pk.job[0] = pack_job(agu_pad, H, r16, H, a_gate, H, r, H, false);
  pk.job[1] = pack_job(agu_pad + size_t(r16) * H * eb, H, r16, H, a_up, H, r, H, false);
  pk.job[2] = pack_job(ad_pad, I, r16, I, a_down, I, r, I, false);
  pk.job[3] = pack_job(bext_g, 2 * r16, I, 2 * r16, b_gate, r, I, r, false);
  pk.job[4] = pack_job(bext_u, 2 * r16, I, r16, nullptr, 0, 0, 0, false);
  pk.job[5] = pack_job(bext_u + size_t(r16) * eb, 2 * r16, I, r16, b_up, r, I, r, false);
  pk.job[6] = pack_job(bext_d, r16, H, r16, b_down, r, H, r, false);
  // for the backward
  pk.job[7] = pack_job(at(saved, SL.bdT), H, r16, H, b_down, r, H, r, true);  // B_d^T
  pk.job[8] = pack_job(at(saved, SL.bgT), I, r16, I, b_gate, r, I, r, true);  // B_g^T
  pk.job[9] = pack_job(at(saved, SL.buT), I, r16, I, b_up, r, I, r, true);    // B_u^T
  pk.njobs = 10;
  LMLP_SIDE_REC("pack(fwd)", SK_PACK, pk, eb, launch_pack(pk, eb, st));
  float* sc_g = d.q4_inkernel ? reinterpret_cast<float*>(at(workspace, FL.sc_g)) : nullptr;
  float* sc_u = d.q4_inkernel ? reinterpret_cast<float*>(at(workspace, FL.sc_u)) : nullptr;
  float* sc_d = d.q4_inkernel ? reinterpret_cast<float*>(at(workspace, FL.sc_d)) : nullptr;
  const void* wg = w_gate;
  const void* wu = w_up;
  const void* wd = w_down;
  if (d.int4 && !d.q4_inkernel) {
    char* wq_g = at(workspace, FL.wq_g);
    char* wq_u = at(workspace, FL.wq_u);
    char* wq_d = at(workspace, FL.wq_d);
    LMLP_SIDE("dequant(W)", launch_dequant_int4(w_gate, w_gate_scales, I, H, wq_g, st));
    LMLP_SIDE("dequant(W)", launch_dequant_int4(w_up, w_up_scales, I, H, wq_u, st));
    LMLP_SIDE("dequant(W)", launch_dequant_int4(w_down, w_down_scales, H, I, wq_d, st));
    wg = wq_g;
    wu = wq_u;
    wd = wq_d;
  }
  if (d.q4_inkernel) {
    ScalePackParams sp{};
    sp.job[0] = {static_cast<const __half*>(w_gate_scales), sc_g, I, H / 64, I};
    sp.job[1] = {static_cast<const __half*>(w_up_scales), sc_u, I, H / 64, I};
    sp.job[2] = {static_cast<const __half*>(w_down_scales), sc_d, H, I / 64, H};
    sp.njobs = 3;
    LMLP_SIDE("pack(scales)", launch_scale_pack(sp, st));
  }

  float* rpp = reinterpret_cast<float*>(at(workspace, FL.rp_part));
  RowProjParams rp{};
  rp.T = T;
  rp.njobs = 1;
  rp.job[0] = rp_job(d, x, H, H, agu_pad, H, int(2 * r16), rpp);
  LMLP_SIDE_REC("rowproj(X A^T)", SK_ROWPROJ, rp, d.bf16, launch_rowproj(rp, d.bf16, st));
  ProjFinishParams fp{};
  fp.T = T;
  fp.njobs = 1;
  fp.job[0] = fin_job(rpp, rp.job[0].kslices, T * 2 * r16, 2 * r16, int(2 * r16), Pgu, 2 * r16, aext_gu, 2 * r16,
                      d.s, nullptr, 0, 0);
  LMLP_SIDE_REC("finish(P_gu)", SK_FINISH, fp, d.bf16, launch_proj_finish(fp, d.bf16, st));

  GemmParams gp{};
  gp.nseg = 2;
  gp.seg[0] = seg(x, H, wg, wu, H, H, d.q4_inkernel, sc_g, sc_u);
  gp.seg[1] = seg(aext_gu, 2 * r16, bext_g, bext_u, 2 * r16, 2 * r16);
  gp.M = T;
  gp.N = I;
  gp.ldc = I;
  gp.c0 = G;
  gp.c1 = U;
  gp.c2 = Z;
  gp.group_m = 8;
  LMLP_GEMM("gemm(gate/up)", gp, 0, EPI_SWIGLU_FWD);

  rp.job[0] = rp_job(d, Z, I, I, ad_pad, I, int(r16), rpp);
  LMLP_SIDE_REC("rowproj(Z A_d^T)", SK_ROWPROJ, rp, d.bf16, launch_rowproj(rp, d.bf16, st));
  fp.job[0] = fin_job(rpp, rp.job[0].kslices, T * r16, r16, int(r16), Pd, r16, aext_d, r16, d.s, nullptr, 0, 0);
  LMLP_SIDE_REC("finish(Pd)", SK_FINISH, fp, d.bf16, launch_proj_finish(fp, d.bf16, st));

  GemmParams gd{};
  gd.nseg = 2;
  gd.seg[0] = seg(Z, I, wd, nullptr, I, I, d.q4_inkernel, sc_d, nullptr);
  gd.seg[1] = seg(aext_d, r16, bext_d, nullptr, r16, r16);
  gd.M = T;
  gd.N = H;
  gd.ldc = H;
  gd.c0 = y;
  gd.group_m = 8;
  if (ex.phase < 0) gd.tile_n = store_tile_n(d, T, H);  // grouped launches keep one tile shape
  LMLP_GEMM("gemm(down)", gd, 0, EPI_STORE);
  return LMLP_OK;
}

// The MLP backward; with LMLP_RMSNORM the normalised rows are re-applied from
// the saved statistics first and dx is carried through the norm at the end.
static int backward_impl(const lmlp_dims* dims, const void* gamma, const void* dy, const void* x,
                         const void* w_gate, const void* w_gate_scales, const void* w_up, const void* w_up_scales,
                         const void* w_down, const void* w_down_scales, const void* a_gate, const void* b_gate,
                         const void* a_up, const void* b_up, const void* a_down, const void* b_down, void* saved,
                         size_t saved_bytes, void* dx, void* da_gate, void* db_gate, void* da_up, void* db_up,
                         void* da_down, void* db_down, void* workspace, size_t workspace_bytes, void* stream,
                         Exec* exec = nullptr) {
  Exec local_exec;
  Exec& ex = exec ? *exec : local_exec;
  Dims d;
  LMLP_TRY(parse_dims(dims, d));
  d.t_split = ex.t_split;
  if (d.norm) LMLP_TRY(need_ptr(gamma, "gamma"));
  LMLP_TRY(check_weights(d, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales));
  LMLP_TRY(check_adapters(a_gate, b_gate, a_up, b_up, a_down, b_down));
  LMLP_TRY(need_ptr(da_gate, "da_gate"));
  LMLP_TRY(need_ptr(db_gate, "db_gate"));
  LMLP_TRY(need_ptr(da_up, "da_up"));
  LMLP_TRY(need_ptr(db_up, "db_up"));
  LMLP_TRY(need_ptr(da_down, "da_down"));
  LMLP_TRY(need_ptr(db_down, "db_down"));
  const SavedLayout SL = saved_layout(d);
  const BwdLayout BL = bwd_layout(d);
  if (d.T > 0) {
    LMLP_TRY(need_ptr(dy, "dy"));
    LMLP_TRY(need_ptr(x, "x"));
    LMLP_TRY(need_ptr(dx, "dx"));
    LMLP_TRY(need_ptr(saved, "saved"));
    LMLP_TRY(need_ptr(workspace, "workspace"));
  }
  if (saved_bytes < SL.total) return fail(LMLP_ERR_WORKSPACE, "saved buffer smaller than lora_mlp_saved_bytes()");
  if (workspace_bytes < BL.total)
    return fail(LMLP_ERR_WORKSPACE, "workspace smaller than lora_mlp_workspace_bytes(dims, 1)");
  LMLP_TRY(check_device());

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t T = d.T, H = d.H, I = d.I, r = d.r, r16 = d.r16;
  const int eb = d.eb;
  const float s = d.s;

  ReduceParams rd{};
  if (T == 0) {
    // no tokens: every adapter gradient is an empty sum
    rd.job[0] = rd_job(nullptr, 0, 0, 0, 0, I, r, db_gate, r, false, s, d.bf16);
    rd.job[1] = rd_job(nullptr, 0, 0, 0, 0, I, r, db_up, r, false, s, d.bf16);
    rd.job[2] = rd_job(nullptr, 0, 0, 0, 0, r, I, da_down, I, false, s, d.bf16);
    rd.job[3] = rd_job(nullptr, 0, 0, 0, 0, r, H, da_gate, H, false, s, d.bf16);
    rd.job[4] = rd_job(nullptr, 0, 0, 0, 0, r, H, da_up, H, false, s, d.bf16);
    rd.job[5] = rd_job(nullptr, 0, 0, 0, 0, H, r, db_down, r, false, s, d.bf16);
    rd.njobs = 6;
    LMLP_SIDE_REC("reduce(zero)", SK_REDUCE, rd, 0, launch_reduce(rd, st));
    return LMLP_OK;
  }

  const void* x_in = x;
  NormParams np{};
  if (d.norm) {  // the forward's normalised rows, from its saved rstd
    np.x = x;
    np.gamma = gamma;
    np.xn = at(workspace, BL.xn);
    np.rstd = reinterpret_cast<float*>(at(saved, SL.rstd));
    np.T = T;
    np.H = H;
    np.mode = NORM_APPLY;
    LMLP_SIDE("rmsnorm(apply)", launch_rmsnorm(np, d.bf16, st));
    x = np.xn;
  }

  char* G_rc = d.recompute ? at(workspace, BL.g_rc) : nullptr;
  char* U_rc = d.recompute ? at(workspace, BL.u_rc) : nullptr;
  const char* G = d.recompute ? G_rc : at(saved, SL.g);
  const char* U = d.recompute ? U_rc : at(saved, SL.u);
  const float* Pgu = reinterpret_cast<const float*>(at(saved, SL.pgu));
  const float* Pd = reinterpret_cast<const float*>(at(saved, SL.pd));
  // dG, dU in place of G, U when those are not needed afterwards
  char* dG = d.recompute ? G_rc : d.consume ? at(saved, SL.g) : at(workspace, BL.dg);
  char* dU = d.recompute ? U_rc : d.consume ? at(saved, SL.u) : at(workspace, BL.du);
  char* Z = at(workspace, BL.z);
  float* Qd = reinterpret_cast<float*>(at(workspace, BL.qd));
  char* aext_d = at(workspace, BL.aext_d);
  float* Qgu = reinterpret_cast<float*>(at(workspace, BL.qgu));
  char* aext_gu = at(workspace, BL.aext_gu);
  // adapter factors packed by the forward
  const char* bdT = at(saved, SL.bdT);
  const char* bgT = at(saved, SL.bgT);
  const char* buT = at(saved, SL.buT);
  const char* ad_pad = at(saved, SL.ad_pad);
  const char* agu_pad = at(saved, SL.agu_pad);
  float* rpa = reinterpret_cast<float*>(at(workspace, BL.rp_a));
  float* rpb = reinterpret_cast<float*>(at(workspace, BL.rp_b));
  const int64_t ldT = ld_tok(d);
  char* pguT = d.bf16 ? at(workspace, BL.pguT) : nullptr;
  char* pdT = d.bf16 ? at(workspace, BL.pdT) : nullptr;
  char* qdT = d.bf16 ? at(workspace, BL.qdT) : nullptr;
  char* qguT = d.bf16 ? at(workspace, BL.qguT) : nullptr;
  float* part_dg = reinterpret_cast<float*>(at(workspace, BL.part_dg));
  float* part_du = reinterpret_cast<float*>(at(workspace, BL.part_du));
  float* part_z = reinterpret_cast<float*>(at(workspace, BL.part_z));
  float* part_x = reinterpret_cast<float*>(at(workspace, BL.part_x));
  float* part_dy = reinterpret_cast<float*>(at(workspace, BL.part_dy));

  const void* wg = w_gate;
  const void* wu = w_up;
  const void* wd = w_down;
  const bool ink = d.q4_inkernel;
  float* scn_g = ink ? reinterpret_cast<float*>(at(workspace, BL.scn_g)) : nullptr;
  float* scn_u = ink ? reinterpret_cast<float*>(at(workspace, BL.scn_u)) : nullptr;
  float* scn_d = ink ? reinterpret_cast<float*>(at(workspace, BL.scn_d)) : nullptr;
  float* sct_g = ink && d.recompute ? reinterpret_cast<float*>(at(workspace, BL.sct_g)) : nullptr;
  float* sct_u = ink && d.recompute ? reinterpret_cast<float*>(at(workspace, BL.sct_u)) : nullptr;
  if (d.int4 && !ink) {
    char* wq_g = at(workspace, BL.wq_g);
    char* wq_u = at(workspace, BL.wq_u);
    char* wq_d = at(workspace, BL.wq_d);
    LMLP_SIDE("dequant(W)", launch_dequant_int4(w_gate, w_gate_scales, I, H, wq_g, st));
    LMLP_SIDE("dequant(W)", launch_dequant_int4(w_up, w_up_scales, I, H, wq_u, st));
    LMLP_SIDE("dequant(W)", launch_dequant_int4(w_down, w_down_scales, H, I, wq_d, st));
    wg = wq_g;
    wu = wq_u;
    wd = wq_d;
  }
  if (ink) {  // scales for the decode inside the GEMM staging
    ScalePackParams sp{};
    sp.job[0] = {static_cast<const __half*>(w_gate_scales), scn_g, I, H / 64, sc_ld4(H), 1, 0};
    sp.job[1] = {static_cast<const __half*>(w_up_scales), scn_u, I, H / 64, sc_ld4(H), 1, 0};
    sp.job[2] = {static_cast<const __half*>(w_down_scales), scn_d, H, I / 64, sc_ld4(I), 1, 0};
    sp.njobs = 3;
    LMLP_SIDE("pack(scales)", launch_scale_pack(sp, st));
    if (d.recompute) {
      ScalePackParams sq{};
      sq.job[0] = {static_cast<const __half*>(w_gate_scales), sct_g, I, H / 64, I, 0, 0};
      sq.job[1] = {static_cast<const __half*>(w_up_scales), sct_u, I, H / 64, I, 0, 0};
      sq.njobs = 2;
      LMLP_SIDE("pack(scales)", launch_scale_pack(sq, st));
    }
  }

  RowProjParams rp{};
  rp.T = T;
  rp.njobs = 1;
  rp.job[0] = rp_job(d, dy, H, H, bdT, H, int(r16), rpa);
  LMLP_SIDE_REC("rowproj(dY B_d)", SK_ROWPROJ, rp, d.bf16, launch_rowproj(rp, d.bf16, st));
  // Q_d, and (bf16) the transposed copies the column projections read
  ProjFinishParams fp{};
  fp.T = T;
  fp.njobs = 1;
  fp.job[0] = fin_job(rpa, rp.job[0].kslices, T * r16, r16, int(r16), Qd, r16, aext_d, r16, s, qdT, ldT, 0);
  if (d.bf16) {
    fp.job[1] = fin_job(Pgu, 1, 0, 2 * r16, int(2 * r16), nullptr, 0, nullptr, 0, 1.f, pguT, ldT, 0);
    fp.job[2] = fin_job(Pd, 1, 0, r16, int(r16), nullptr, 0, nullptr, 0, 1.f, pdT, ldT, 0);
    fp.njobs = 3;
  }
  if (d.recompute)  // s P_gu in the compute dtype: the gate/up product's adapter segment
    fp.job[fp.njobs++] = fin_job(Pgu, 1, 0, 2 * r16, int(2 * r16), nullptr, 0, aext_gu, 2 * r16, s, nullptr, 0, 0);
  LMLP_SIDE_REC("finish(Q_d, P^T)", SK_FINISH, fp, d.bf16, launch_proj_finish(fp, d.bf16, st));

  if (d.recompute) {
    // G, U again from X: the forward's gate/up product (its adapter segment
    // from the saved P_gu, bit for bit the forward's), without Z. aext_gu is
    // free until finish(Q_gu) overwrites it.
    GemmParams gp{};
    gp.nseg = 2;
    gp.seg[0] = seg(x, H, wg, wu, H, H, ink, sct_g, sct_u);
    gp.seg[1] = seg(aext_gu, 2 * r16, at(saved, SL.bext_g), at(saved, SL.bext_u), 2 * r16, 2 * r16);
    gp.M = T;
    gp.N = I;
    gp.ldc = I;
    gp.c0 = G_rc;
    gp.c1 = U_rc;
    gp.c2 = nullptr;
    gp.group_m = 8;
    LMLP_GEMM("gemm(gate/up, recompute)", gp, 0, EPI_SWIGLU_FWD);
  }

  GemmParams gz{};
  gz.nseg = 2;
  gz.seg[0] = seg(dy, H, wd, nullptr, I, H, ink, scn_d, nullptr);
  gz.seg[1] = seg(aext_d, r16, ad_pad, nullptr, I, r16);
  gz.M = T;
  gz.N = I;
  gz.ldc = I;
  gz.c0 = dG;
  gz.c1 = dU;
  gz.c2 = Z;
  gz.g_in = G;
  gz.u_in = U;
  gz.group_m = 8;
  int q_parts = 0;
  if (fused_q(d)) {  // Q_g, Q_u partials from the dZ epilogue
    gz.pj_b0 = bgT;
    gz.pj_b1 = buT;
    gz.pj_part0 = rpa;
    gz.pj_part1 = rpb;
    gz.pj_ldb = I;
    gz.pj_T = T;
    gz.pj_r16 = int(r16);
    gz.pj_pguT = pguT;
    gz.pj_qdT = qdT;
    gz.pj_ldt = ldT;
    gz.pj_cdg = part_dg;
    gz.pj_cdu = part_du;
    gz.pj_cz = part_z;
    gz.pj_ncol = I;
    gz.c2 = nullptr;  // Z is only needed for Q_d^T Z, formed here
  }
  // columns in 256-wide tiles; grouped launches balance over the experts, and
  // one split for all of them keeps their phases aligned
  const int64_t n1 = ex.phase < 0 && !ink ? dz_split(d) : d.I;
  if (n1 > 0) {
    GemmParams g1 = gz;
    g1.N = n1;
    LMLP_GEMM("gemm(dZ)", g1, 1, EPI_SWIGLU_BWD);
  }
  if (n1 < I) {  // the tail columns in 128-wide tiles
    GemmParams g2 = gz;
    g2.N = I - n1;
    g2.tile_n = 128;
    g2.seg[0].b0 = static_cast<const char*>(wd) + n1 * eb;
    g2.seg[1].b0 = ad_pad + n1 * eb;
    g2.c0 = dG + n1 * eb;
    g2.c1 = dU + n1 * eb;
    if (g2.c2) g2.c2 = Z + n1 * eb;
    g2.g_in = G + n1 * eb;
    g2.u_in = U + n1 * eb;
    if (fused_q(d)) {
      g2.pj_b0 = bgT + n1 * eb;
      g2.pj_b1 = buT + n1 * eb;
      g2.pj_cdg = part_dg + n1 * 16;
      g2.pj_cdu = part_du + n1 * 16;
      g2.pj_cz = part_z + n1 * 16;
      g2.pj_slice0 = int(n1 / 256);
    }
    LMLP_GEMM("gemm(dZ tail)", g2, 1, EPI_SWIGLU_BWD);
  }
  if (fused_q(d)) q_parts = int((n1 + 255) / 256 + (I - n1 + 127) / 128);

  if (!fused_q(d)) {
    rp.njobs = 2;
    rp.job[0] = rp_job(d, dG, I, I, bgT, I, int(r16), rpa);
    rp.job[1] = rp_job(d, dU, I, I, buT, I, int(r16), rpb);
    LMLP_SIDE_REC("rowproj(dG B_g, dU B_u)", SK_ROWPROJ, rp, d.bf16, launch_rowproj(rp, d.bf16, st));
    q_parts = rp.job[0].kslices;
  }
  fp.njobs = 2;
  fp.job[0] = fin_job(rpa, q_parts, T * r16, r16, int(r16), Qgu, 2 * r16, aext_gu, 2 * r16, s, qguT, ldT, 0);
  fp.job[1] = fin_job(rpb, q_parts, T * r16, r16, int(r16), Qgu, 2 * r16, aext_gu, 2 * r16, s, qguT, ldT,
                      int(r16));
  LMLP_SIDE_REC("finish(Q_gu)", SK_FINISH, fp, d.bf16, launch_proj_finish(fp, d.bf16, st));

  GemmParams gx{};
  gx.nseg = 3;
  gx.seg[0] = seg(dG, I, wg, nullptr, H, I, ink, scn_g, nullptr);
  gx.seg[1] = seg(dU, I, wu, nullptr, H, I, ink, scn_u, nullptr);
  gx.seg[2] = seg(aext_gu, 2 * r16, agu_pad, nullptr, H, 2 * r16);
  gx.M = T;
  gx.N = H;
  gx.ldc = H;
  gx.c0 = dx;
  gx.group_m = 8;
  if (ex.phase < 0) gx.tile_n = store_tile_n(d, T, H);
  LMLP_GEMM("gemm(dX)", gx, 1, EPI_STORE);

  const int ntb = BL.ntb;
  const int64_t tr = BL.tr;
  ColProjParams cp{};
  cp.T = T;
  const size_t trow = size_t(ldT) * eb;  // bytes of one transposed row
  cp.job[0] = cp_job(d, x, H, H, Qgu, 2 * r16, qguT, ldT, int(2 * r16), part_x, ntb, tr);
  cp.job[1] = cp_job(d, dy, H, H, Pd, r16, pdT, ldT, int(r16), part_dy, ntb, tr);
  cp.njobs = 2;
  int nsl_i = int(col_slices(d));  // slices of the [I]-side partials
  if (!fused_q(d)) {
    cp.job[2] = cp_job(d, dG, I, I, Pgu, 2 * r16, pguT, ldT, int(r16), part_dg, ntb, tr);
    cp.job[3] = cp_job(d, dU, I, I, Pgu + r16, 2 * r16, pguT ? pguT + r16 * trow : nullptr, ldT, int(r16), part_du,
                       ntb, tr);
    cp.job[4] = cp_job(d, Z, I, I, Qd, r16, qdT, ldT, int(r16), part_z, ntb, tr);
    cp.njobs = 5;
    nsl_i = ntb;
  }
  LMLP_SIDE_REC("colproj", SK_COLPROJ, cp, d.bf16, launch_colproj(cp, d.bf16, st));

  rd.job[0] = rd_job(part_dg, I * r16, nsl_i, r16, 0, I, r, db_gate, r, false, s, d.bf16);
  rd.job[1] = rd_job(part_du, I * r16, nsl_i, r16, 0, I, r, db_up, r, false, s, d.bf16);
  rd.job[2] = rd_job(part_z, I * r16, nsl_i, r16, 0, I, r, da_down, I, true, s, d.bf16);
  rd.job[3] = rd_job(part_x, H * 2 * r16, ntb, 2 * r16, 0, H, r, da_gate, H, true, s, d.bf16);
  rd.job[4] = rd_job(part_x, H * 2 * r16, ntb, 2 * r16, int(r16), H, r, da_up, H, true, s, d.bf16);
  rd.job[5] = rd_job(part_dy, H * r16, ntb, r16, 0, H, r, db_down, r, false, s, d.bf16);
  rd.njobs = 6;
  LMLP_SIDE_REC("reduce", SK_REDUCE, rd, 0, launch_reduce(rd, st));
  if (d.norm) {  // dx (so far the gradient of the normalised rows) through the norm, in place
    np.x = x_in;
    np.g = dx;
    np.dx = dx;
    np.mode = NORM_BWD;
    LMLP_SIDE("rmsnorm(bwd)", launch_rmsnorm(np, d.bf16, st));
  }
  return LMLP_OK;
}

int lora_mlp_forward(const lmlp_dims* dims, const void* x, const void* w_gate, const void* w_gate_scales,
                     const void* w_up, const void* w_up_scales, const void* w_down, const void* w_down_scales,
                     const void* a_gate, const void* b_gate, const void* a_up, const void* b_up,
                     const void* a_down, const void* b_down, void* y, void* saved, size_t saved_bytes,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (dims && (dims->flags & LMLP_RMSNORM))
    return fail(LMLP_ERR_INVALID_ARG, "LMLP_RMSNORM is for lora_mlp_norm_forward");
  return forward_impl(dims, nullptr, 0.f, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                      a_gate, b_gate, a_up, b_up, a_down, b_down, y, saved, saved_bytes, workspace, workspace_bytes,
                      stream);
}

int lora_mlp_backward(const lmlp_dims* dims, const void* dy, const void* x, const void* w_gate,
                      const void* w_gate_scales, const void* w_up, const void* w_up_scales, const void* w_down,
                      const void* w_down_scales, const void* a_gate, const void* b_gate, const void* a_up,
                      const void* b_up, const void* a_down, const void* b_down, void* saved, size_t saved_bytes,
                      void* dx, void* da_gate, void* db_gate, void* da_up, void* db_up, void* da_down,
                      void* db_down, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (dims && (dims->flags & LMLP_RMSNORM))
    return fail(LMLP_ERR_INVALID_ARG, "LMLP_RMSNORM is for lora_mlp_norm_backward");
  return backward_impl(dims, nullptr, dy, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales,
                       a_gate, b_gate, a_up, b_up, a_down, b_down, saved, saved_bytes, dx, da_gate, db_gate, da_up,
                       db_up, da_down, db_down, workspace, workspace_bytes, stream);
}

int lora_mlp_norm_forward(const lmlp_dims* dims, float eps, const void* x, const void* gamma, const void* w_gate,
                          const void* w_gate_scales, const void* w_up, const void* w_up_scales, const void* w_down,
                          const void* w_down_scales, const void* a_gate, const void* b_gate, const void* a_up,
                          const void* b_up, const void* a_down, const void* b_down, void* y, void* saved,
                          size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (dims && !(dims->flags & LMLP_RMSNORM))
    return fail(LMLP_ERR_INVALID_ARG, "lora_mlp_norm_forward needs LMLP_RMSNORM in dims.flags");
  if (!std::isfinite(eps) || eps < 0.f) return fail(LMLP_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return forward_impl(dims, gamma, eps, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales, a_gate,
                      b_gate, a_up, b_up, a_down, b_down, y, saved, saved_bytes, workspace, workspace_bytes, stream);
}

int lora_mlp_norm_backward(const lmlp_dims* dims, const void* dy, const void* x, const void* gamma,
                           const void* w_gate, const void* w_gate_scales, const void* w_up, const void* w_up_scales,
                           const void* w_down, const void* w_down_scales, const void* a_gate, const void* b_gate,
                           const void* a_up, const void* b_up, const void* a_down, const void* b_down, void* saved,
                           size_t saved_bytes, void* dx, void* da_gate, void* db_gate, void* da_up, void* db_up,
                           void* da_down, void* db_down, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (dims && !(dims->flags & LMLP_RMSNORM))
    return fail(LMLP_ERR_INVALID_ARG, "lora_mlp_norm_backward needs LMLP_RMSNORM in dims.flags");
  return backward_impl(dims, gamma, dy, x, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales, a_gate,
                       b_gate, a_up, b_up, a_down, b_down, saved, saved_bytes, dx, da_gate, db_gate, da_up, db_up,
                       da_down, db_down, workspace, workspace_bytes, stream);
}

// ---- grouped (MoE) LoRA MLP -------------------------------------------------
// Rows grouped by expert (host offsets); per-expert tensors stacked along a
// leading axis. Every argument is checked for all experts before anything is
// enqueued; then each expert runs the fused MLP above on its rows and its
// slices of the stacked tensors, in phases cut at the GEMMs (Exec): in each
// phase the experts' side kernels (packing, row projections and their
// finishes, column projections, reduce) go out merged across experts, one
// launch per kind and round with one job per expert and the expert's own
// token count, and then the GEMMs they lead to run as one grouped launch per
// kind over all experts' tiles (a few hundred rows per expert are only tens
// of tiles for 256 CUs). Everything runs on the caller's stream. `saved` and
// the workspace hold one region per expert, in expert order, so every
// expert's intermediates stay resident across the phases. An expert without
// rows gets zero adapter gradients. Each expert's arithmetic is that of the
// plain entry point, so results are bitwise reproducible.


struct MoePlan {
  std::vector<lmlp_dims> dims;  // per expert: tokens = its rows
  std::vector<int64_t> row0;
  std::vector<size_t> soff, ssize;          // saved region of each expert
  std::vector<size_t> wfoff, wfsize, wboff, wbsize;  // forward / backward workspace regions
  size_t saved_total = 0, ws_fwd = 0, ws_bwd = 0;
  // one region per pass for the tables of a phase (more experts than one
  // launch's arguments hold): GEMM parameter blocks and side-kernel jobs
  size_t tab_fwd = 0, tab_bwd = 0, tab_bytes = 0;
  bool table = false;
  // K splits of the grouped down (forward) and dX (backward) products, with
  // their fp32 partials [S][tokens][H] in the workspace (1: no split)
  int split_down = 1, split_dx = 1;
  size_t part_fwd = 0, part_bwd = 0;
  Dims d;  // the whole call
};

// Run the passes body(e, exec) of the experts in `order` phase by phase, all
// on the caller's stream: in each phase every expert records its batchable
// side kernels (its other side launches, the 4-bit decode and scale packing,
// go out at once: only GEMMs read what they write), the recorded launches go
// out merged across experts round by round (round r: every expert's r-th
// launch; one expert's launches keep their order), then the GEMMs the
// experts reached, grouped by kind; until no expert hands back a GEMM.
// The job and parameter tables of one pass of the grouped MLP, in one
// batch: laid out back to back (256-byte aligned) in a host buffer whose
// device copy is the pass's table region of the workspace, with the launches
// that read them queued; flush() stages the buffer with one read of the
// pinned ring and then enqueues the launches in order, each timed under its
// name when profiling is on.
class PhaseTables final : public TableBatch {
 public:
  PhaseTables(void* dev, size_t cap, hipStream_t st) : dev_(static_cast<char*>(dev)), cap_(cap), st_(st) {}
  const char* name = "";  // of the launches deferred next
  void* add(const void* src, size_t bytes) override {
    const size_t off = (host_.size() + 255) / 256 * 256;
    if (off + bytes > cap_) return nullptr;
    host_.resize(off + bytes);
    std::memcpy(host_.data() + off, src, bytes);
    return dev_ + off;
  }
  void defer(std::function<hipError_t()> launch) override { q_.push_back({name, std::move(launch)}); }
  hipError_t make_room() override {
    failed_ = nullptr;
    return run();
  }
  int flush() {
    failed_ = nullptr;
    const hipError_t e = run();
    return e == hipSuccess ? LMLP_OK : hip_rc(e, failed_ ? failed_ : "tables");
  }

 private:
  hipError_t run() {
    hipStream_t st = st_;
    if (!host_.empty()) {
      ProfScope ps(st, "tables");
      const hipError_t e = stage_device_table(host_.data(), host_.size(), dev_, st);
      if (e != hipSuccess) return e;
      ps.done();
    }
    for (auto& l : q_) {
      ProfScope ps(st, l.first);
      const hipError_t e = l.second();
      if (e != hipSuccess) {
        failed_ = l.first;
        return e;
      }
      ps.done();
    }
    host_.clear();
    q_.clear();
    return hipSuccess;
  }
  char* dev_;
  size_t cap_;
  hipStream_t st_;
  std::vector<char> host_;
  std::vector<std::pair<const char*, std::function<hipError_t()>>> q_;
  const char* failed_ = nullptr;
};

// A grouped product of the plain store kind run as S splits of K, each
// expert's split s storing fp32 partials at its rows of part[s], then one
// ordered sum over all rows into `out` (the experts' row blocks tile it).
struct MoeSplitK {
  const char* name = nullptr;  // the GEMM kind
  int S = 1;
  float* part = nullptr;  // [S][rows][N]
  void* out = nullptr;    // [rows][N], bf16
  int64_t rows = 0, N = 0;
};

// Split s of a plain-store product (256-wide tiles) over K: the down
// product's one large segment is cut in two at a multiple of 32 (the
// adapter segment goes with the second half); dX's two large segments (dG
// W_g, dU W_u) go one to each split, the adapter with the second.
static GemmParams split_params(const GemmParams& g, int s, int nn) {
  GemmParams q = g;
  if (nn) {  // dX: seg 0 | seg 1 + seg 2
    if (s == 0) {
      q.nseg = 1;
      q.seg[1] = q.seg[2] = GemmSeg{};
    } else {
      q.nseg = g.nseg - 1;
      q.seg[0] = g.seg[1];
      q.seg[1] = g.seg[2];
      q.seg[2] = GemmSeg{};
    }
    return q;
  }
  const int64_t kh = g.seg[0].K / 64 * 32;  // first half, a multiple of 32
  if (s == 0) {
    q.nseg = 1;
    q.seg[0].K = kh;
    q.seg[1] = q.seg[2] = GemmSeg{};
  } else {
    q.seg[0].a = static_cast<const uint16_t*>(g.seg[0].a) + kh;    // bf16 elements
    q.seg[0].b0 = static_cast<const uint16_t*>(g.seg[0].b0) + kh;  // NT: K contiguous in B's rows
    q.seg[0].K = g.seg[0].K - kh;
  }
  return q;
}

static int moe_phased(hipStream_t caller, const std::vector<int64_t>& order, int64_t t_split, void* tables,
                      size_t table_bytes, const std::function<int(int64_t, Exec*, hipStream_t)>& body,
                      const MoeSplitK& split = MoeSplitK{}) {
  std::vector<Exec> ex(order.size());
  std::vector<std::vector<SideOp>> ops(order.size());
  hipStream_t st = caller;
  // one batch for the whole pass: its phases are recorded one after another
  // (the host plans them without the device), their launches queued in order,
  // and the tables read with one fetch (more when they outgrow the region)
  PhaseTables tb(tables, table_bytes, st);
  PhaseTables* tbp = tables ? &tb : nullptr;
  for (int phase = 0;; ++phase) {
    size_t rounds = 0;
    for (size_t k = 0; k < order.size(); ++k) {
      ex[k] = Exec{};
      ex[k].t_split = t_split;
      ex[k].phase = phase;
      ops[k].clear();
      ex[k].rec = &ops[k];
      LMLP_TRY(body(order[k], &ex[k], caller));
      rounds = std::max(rounds, ops[k].size());
    }
    for (size_t r = 0; r < rounds; ++r) {
      std::vector<bool> taken(order.size(), false);
      for (size_t k = 0; k < order.size(); ++k) {
        if (taken[k] || r >= ops[k].size()) continue;
        const SideOp& a = ops[k][r];
        std::vector<const SideOp*> grp;
        for (size_t j = k; j < order.size(); ++j) {
          if (taken[j] || r >= ops[j].size()) continue;
          const SideOp& b = ops[j][r];
          if (b.kind != a.kind || b.flag != a.flag || std::strcmp(b.name, a.name) != 0) continue;
          grp.push_back(&b);
          taken[j] = true;
        }
        if (tbp) {
          tb.name = a.name;
          LMLP_TRY(hip_rc(launch_side_group(grp, st, tbp), a.name));
        } else {
          LMLP_LAUNCH(a.name, launch_side_group(grp, st, nullptr));
        }
      }
    }
    // the GEMMs of this phase: dense bf16 ones grouped by kind, the rest one by one
    bool any = false;
    std::vector<bool> done(order.size(), false);
    for (size_t k = 0; k < order.size(); ++k) {
      if (!ex[k].sunk || done[k]) continue;
      any = true;
      if (!ex[k].groupable) {
        const GemmParams gp = ex[k].gp;
        const int nn = ex[k].nn, epi = ex[k].epi;
        auto one = [gp, nn, epi, st]() {
          return gp.seg[0].bint4 ? run_q4(gp, nn, epi, st) : launch_gemm_f32(gp, nn, epi, st);
        };
        if (tbp) {
          tb.name = ex[k].name;
          tb.defer(one);
        } else {
          LMLP_LAUNCH(ex[k].name, one());
        }
        done[k] = true;
        continue;
      }
      std::vector<GemmParams> grp;
      for (size_t j = k; j < order.size(); ++j) {
        const Exec& a = ex[k];
        const Exec& b = ex[j];
        if (done[j] || !b.sunk || !b.groupable || std::strcmp(a.name, b.name) != 0 || a.nn != b.nn ||
            a.epi != b.epi || a.gp.tile_n != b.gp.tile_n || (a.gp.pj_part0 == nullptr) != (b.gp.pj_part0 == nullptr))
          continue;
        grp.push_back(b.gp);
        done[j] = true;
      }
      // largest products first: workgroups start in order, so the longest
      // groups begin early and the last wave is made of short ones
      std::stable_sort(grp.begin(), grp.end(), [](const GemmParams& x, const GemmParams& y) { return x.M > y.M; });
      const int nn = ex[k].nn, epi = ex[k].epi;
      if (tbp && split.S > 1 && epi == EPI_STORE && std::strcmp(ex[k].name, split.name) == 0) {
        // every expert's S splits in one table launch (largest first), then the sum
        std::vector<GemmParams> sg;
        for (const GemmParams& g : grp) {
          const int64_t row = (static_cast<const char*>(g.c0) - static_cast<const char*>(split.out)) /
                              static_cast<int64_t>(split.N * sizeof(uint16_t));
          for (int sp = 0; sp < split.S; ++sp) {
            GemmParams q = split_params(g, sp, nn);
            q.c0 = split.part + (sp * split.rows + row) * split.N;
            q.tile_n = 0;
            sg.push_back(q);
          }
        }
        std::stable_sort(sg.begin(), sg.end(), [](const GemmParams& x, const GemmParams& y) { return x.M > y.M; });
        tb.name = ex[k].name;
        LMLP_TRY(hip_rc(launch_gemm_bf16_grouped_table(sg.data(), int(sg.size()), nn, EPI_STORE_F32, nullptr, st, tbp),
                        ex[k].name));
        const MoeSplitK sk = split;
        tb.name = nn ? "sum(dX)" : "sum(down)";
        tb.defer([sk, st]() { return launch_splitk_sum(sk.part, sk.S, sk.rows * sk.N, sk.out, st); });
      } else if (tbp && grp.size() > size_t(kMaxGemmGroups)) {  // parameter blocks through the phase's tables
        tb.name = ex[k].name;
        LMLP_TRY(hip_rc(launch_gemm_bf16_grouped_table(grp.data(), int(grp.size()), nn, epi, nullptr, st, tbp),
                        ex[k].name));
      } else if (tbp) {
        tb.name = ex[k].name;
        tb.defer([grp, nn, epi, st]() { return launch_gemm_bf16_grouped(grp.data(), int(grp.size()), nn, epi, st); });
      } else {
        LMLP_LAUNCH(ex[k].name, launch_gemm_bf16_grouped(grp.data(), int(grp.size()), nn, epi, st));
      }
    }
    if (!any) break;
  }
  if (tbp) LMLP_TRY(tb.flush());
  return LMLP_OK;
}

static int moe_plan(const lmlp_dims* dims, int64_t E, const int64_t* off, MoePlan& P) {
  LMLP_TRY(parse_dims(dims, P.d));
  if (P.d.norm) return fail(LMLP_ERR_INVALID_ARG, "LMLP_RMSNORM is not supported by the grouped MLP");
  if (E < 1 || E > 65536) return fail(LMLP_ERR_INVALID_ARG, "n_experts must be in [1, 65536]");
  if (!off) return fail(LMLP_ERR_INVALID_ARG, "offsets is NULL");
  if (off[0] != 0 || off[E] != P.d.T) return fail(LMLP_ERR_INVALID_ARG, "offsets must run from 0 to dims.tokens");
  P.dims.resize(E);
  P.row0.resize(E);
  P.soff.resize(E);
  P.ssize.resize(E);
  P.wfoff.resize(E);
  P.wfsize.resize(E);
  P.wboff.resize(E);
  P.wbsize.resize(E);
  for (int64_t e = 0; e < E; ++e) {
    if (off[e + 1] < off[e]) return fail(LMLP_ERR_INVALID_ARG, "offsets must not decrease");
    lmlp_dims de = *dims;
    de.tokens = off[e + 1] - off[e];
    Dims dd;
    LMLP_TRY(parse_dims(&de, dd));
    dd.t_split = P.d.T;
    P.dims[e] = de;
    P.row0[e] = off[e];
    P.soff[e] = P.saved_total;
    P.ssize[e] = saved_layout(dd).total;
    P.saved_total += P.ssize[e];
    P.wfoff[e] = P.ws_fwd;
    P.wfsize[e] = dd.T > 0 ? fwd_layout(dd).total : 0;  // no forward work without rows
    P.ws_fwd += P.wfsize[e];
    // an expert without rows only writes zero gradients: it gets no region
    // (its pass is handed the size it checks, and no pointer)
    P.wboff[e] = P.ws_bwd;
    P.wbsize[e] = bwd_layout(dd).total;
    P.ws_bwd += dd.T > 0 ? P.wbsize[e] : 0;
  }
  // K splits of the grouped down and dX products (few large experts, dense
  // bf16 weights): when their 256 x 256 tiles leave the last wave at most
  // half full, two splits over K double the tiles (e.g. 592 -> 1184 tiles,
  // 2.3 -> 4.6 waves on 256 compute units) at the cost of fp32 partials and
  // their sum, which pays only for long K: at the Mixtral-8x7B shape dX (K =
  // 2I = 28672) went 2.10 -> 1.96 ms with its sum, down (K = I = 14336)
  // 1.03 -> 1.04 ms. So a product splits when its K is at least 16384.
  if (E <= kMaxGemmGroups && P.d.bf16 && !P.d.int4 && P.d.H % 4 == 0) {
    int64_t tiles = 0;
    for (int64_t e = 0; e < E; ++e) tiles += (off[e + 1] - off[e] + 255) / 256 * ((P.d.H + 255) / 256);
    const int64_t ncu = device_cus();
    const int64_t rem = tiles % ncu;
    if (tiles > ncu && rem > 0 && 2 * rem <= ncu) {
      const size_t pb = align_up(size_t(2) * P.d.T * P.d.H * sizeof(float));
      if (P.d.I >= 16384) {
        P.split_down = 2;
        P.part_fwd = P.ws_fwd;
        P.ws_fwd += pb;
      }
      if (2 * P.d.I >= 16384) {
        P.split_dx = 2;
        P.part_bwd = P.ws_bwd;
        P.ws_bwd += pb;
      }
    }
  }
  P.table = E > kMaxGemmGroups || P.split_down > 1 || P.split_dx > 1;
  if (P.table) {
    // a pass's tables: room for four GEMM kinds' parameter blocks and four
    // side launches of kSideJobsPerExpert jobs per expert each; a pass that
    // needs more stages its tables in more than one batch
    P.tab_bytes = 4 * (align_up(size_t(E) * sizeof(GemmParams)) +
                       align_up(size_t(E) * kSideJobsPerExpert * kSideJobBytes));
    P.tab_fwd = P.ws_fwd;
    P.ws_fwd += P.tab_bytes;
    P.tab_bwd = P.ws_bwd;
    P.ws_bwd += P.tab_bytes;
  }
  return LMLP_OK;
}

// bytes between consecutive experts of each stacked tensor
struct MoeStrides {
  size_t wgu, wgu_s, wd, wd_s, agu, bgu, ad, bd, rows;
};
static MoeStrides moe_strides(const Dims& d) {
  MoeStrides S;
  const size_t H = size_t(d.H), I = size_t(d.I), r = size_t(d.r), eb = size_t(d.eb);
  S.wgu = d.int4 ? I * H / 2 : I * H * eb;
  S.wgu_s = d.int4 ? I * (H / 64) * 2 : 0;
  S.wd = d.int4 ? H * I / 2 : H * I * eb;
  S.wd_s = d.int4 ? H * (I / 64) * 2 : 0;
  S.agu = r * H * eb;
  S.bgu = I * r * eb;
  S.ad = r * I * eb;
  S.bd = H * r * eb;
  S.rows = H * eb;  // one token row of x, y, dy, dx
  return S;
}

// item e of a stacked tensor (NULL stays NULL)
static const void* slice(const void* base, int64_t e, size_t stride) {
  return base ? static_cast<const char*>(base) + size_t(e) * stride : nullptr;
}
static void* slice(void* base, int64_t e, size_t stride) {
  return base ? static_cast<char*>(base) + size_t(e) * stride : nullptr;
}

size_t lora_moe_saved_bytes(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets) {
  MoePlan P;
  if (moe_plan(dims, n_experts, offsets, P) != LMLP_OK) return 0;
  return P.saved_total;
}

size_t lora_moe_workspace_bytes(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets,
                                int is_backward) {
  MoePlan P;
  if (moe_plan(dims, n_experts, offsets, P) != LMLP_OK) return 0;
  return is_backward ? P.ws_bwd : P.ws_fwd;
}

int lora_moe_forward(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets, const void* x,
                     const void* w_gate, const void* w_gate_scales, const void* w_up, const void* w_up_scales,
                     const void* w_down, const void* w_down_scales, const void* a_gate, const void* b_gate,
                     const void* a_up, const void* b_up, const void* a_down, const void* b_down, void* y,
                     void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  MoePlan P;
  LMLP_TRY(moe_plan(dims, n_experts, offsets, P));
  const Dims& d = P.d;
  LMLP_TRY(check_weights(d, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales));
  LMLP_TRY(check_adapters(a_gate, b_gate, a_up, b_up, a_down, b_down));
  if (d.T > 0) {
    LMLP_TRY(need_ptr(x, "x"));
    LMLP_TRY(need_ptr(y, "y"));
    LMLP_TRY(need_ptr(saved, "saved"));
    LMLP_TRY(need_ptr(workspace, "workspace"));
  }
  if (saved_bytes < P.saved_total) return fail(LMLP_ERR_WORKSPACE, "saved buffer smaller than lora_moe_saved_bytes()");
  if (workspace_bytes < P.ws_fwd)
    return fail(LMLP_ERR_WORKSPACE, "workspace smaller than lora_moe_workspace_bytes(dims, ..., 0)");
  LMLP_TRY(check_device());
  const MoeStrides S = moe_strides(d);
  std::vector<int64_t> order;  // experts with rows
  for (int64_t e = 0; e < n_experts; ++e)
    if (P.dims[e].tokens > 0) order.push_back(e);
  if (order.empty()) return LMLP_OK;
  void* tab = P.table ? at(workspace, P.tab_fwd) : nullptr;
  MoeSplitK sk;
  if (P.split_down > 1) {
    sk.name = "gemm(down)";
    sk.S = P.split_down;
    sk.part = reinterpret_cast<float*>(at(workspace, P.part_fwd));
    sk.out = y;
    sk.rows = P.d.T;
    sk.N = P.d.H;
  }
  return moe_phased(static_cast<hipStream_t>(stream), order, P.d.T, tab, P.tab_bytes,
                    [&](int64_t e, Exec* ex, hipStream_t ws) {
    return forward_impl(&P.dims[e], nullptr, 0.f, slice(x, P.row0[e], S.rows), slice(w_gate, e, S.wgu),
                        slice(w_gate_scales, e, S.wgu_s), slice(w_up, e, S.wgu), slice(w_up_scales, e, S.wgu_s),
                        slice(w_down, e, S.wd), slice(w_down_scales, e, S.wd_s), slice(a_gate, e, S.agu),
                        slice(b_gate, e, S.bgu), slice(a_up, e, S.agu), slice(b_up, e, S.bgu), slice(a_down, e, S.ad),
                        slice(b_down, e, S.bd), slice(y, P.row0[e], S.rows), at(saved, P.soff[e]), P.ssize[e],
                        at(workspace, P.wfoff[e]), P.wfsize[e], ws, ex);
  }, sk);
}

int lora_moe_backward(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets, const void* dy,
                      const void* x, const void* w_gate, const void* w_gate_scales, const void* w_up,
                      const void* w_up_scales, const void* w_down, const void* w_down_scales, const void* a_gate,
                      const void* b_gate, const void* a_up, const void* b_up, const void* a_down,
                      const void* b_down, void* saved, size_t saved_bytes, void* dx, void* da_gate, void* db_gate,
                      void* da_up, void* db_up, void* da_down, void* db_down, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  MoePlan P;
  LMLP_TRY(moe_plan(dims, n_experts, offsets, P));
  const Dims& d = P.d;
  LMLP_TRY(check_weights(d, w_gate, w_gate_scales, w_up, w_up_scales, w_down, w_down_scales));
  LMLP_TRY(check_adapters(a_gate, b_gate, a_up, b_up, a_down, b_down));
  LMLP_TRY(need_ptr(da_gate, "da_gate"));
  LMLP_TRY(need_ptr(db_gate, "db_gate"));
  LMLP_TRY(need_ptr(da_up, "da_up"));
  LMLP_TRY(need_ptr(db_up, "db_up"));
  LMLP_TRY(need_ptr(da_down, "da_down"));
  LMLP_TRY(need_ptr(db_down, "db_down"));
  if (d.T > 0) {
    LMLP_TRY(need_ptr(dy, "dy"));
    LMLP_TRY(need_ptr(x, "x"));
    LMLP_TRY(need_ptr(dx, "dx"));
    LMLP_TRY(need_ptr(saved, "saved"));
    LMLP_TRY(need_ptr(workspace, "workspace"));
  }
  if (saved_bytes < P.saved_total) return fail(LMLP_ERR_WORKSPACE, "saved buffer smaller than lora_moe_saved_bytes()");
  if (workspace_bytes < P.ws_bwd)
    return fail(LMLP_ERR_WORKSPACE, "workspace smaller than lora_moe_workspace_bytes(dims, ..., 1)");
  LMLP_TRY(check_device());
  const MoeStrides S = moe_strides(d);
  std::vector<int64_t> order(n_experts);  // every expert: one without rows gets zero gradients
  for (int64_t e = 0; e < n_experts; ++e) order[e] = e;
  void* tab = P.table ? at(workspace, P.tab_bwd) : nullptr;
  MoeSplitK sk;
  if (P.split_dx > 1) {
    sk.name = "gemm(dX)";
    sk.S = P.split_dx;
    sk.part = reinterpret_cast<float*>(at(workspace, P.part_bwd));
    sk.out = dx;
    sk.rows = P.d.T;
    sk.N = P.d.H;
  }
  return moe_phased(static_cast<hipStream_t>(stream), order, P.d.T, tab, P.tab_bytes,
                    [&](int64_t e, Exec* ex, hipStream_t ws) {
    const bool any = P.dims[e].tokens > 0;
    return backward_impl(
        &P.dims[e], nullptr, any ? slice(dy, P.row0[e], S.rows) : nullptr, any ? slice(x, P.row0[e], S.rows) : nullptr,
        slice(w_gate, e, S.wgu), slice(w_gate_scales, e, S.wgu_s), slice(w_up, e, S.wgu),
        slice(w_up_scales, e, S.wgu_s), slice(w_down, e, S.wd), slice(w_down_scales, e, S.wd_s),
        slice(a_gate, e, S.agu), slice(b_gate, e, S.bgu), slice(a_up, e, S.agu), slice(b_up, e, S.bgu),
        slice(a_down, e, S.ad), slice(b_down, e, S.bd), any ? at(saved, P.soff[e]) : nullptr, P.ssize[e],
        any ? slice(dx, P.row0[e], S.rows) : nullptr, slice(da_gate, e, S.agu), slice(db_gate, e, S.bgu),
        slice(da_up, e, S.agu), slice(db_up, e, S.bgu), slice(da_down, e, S.ad), slice(db_down, e, S.bd),
        any ? at(workspace, P.wboff[e]) : nullptr, P.wbsize[e], ws, ex);
  }, sk);
}

// ---- fused LoRA linear ----------------------------------------------------
// Forward: pack A, B; rowproj P = x A^T (split-K) and its finish (P fp32 and
// its bf16 transpose to saved, s P as the adapter segment); gemm y = [x | sP]
// [W | B]^T. Backward: rowproj Q = dy B and its finish; gemm dX = [dy | sQ]
// [W ; A] (NN); colproj x^T Q and dy^T P per token block; reduce to
// da = s Q^T x, db = s dy^T P. The same kernels as the MLP's F1/F4, B1/B4,
// B5 and B3 steps.

size_t lora_linear_saved_bytes(const lmlp_dims* dims) {
  Dims d;
  if (parse_linear_dims(dims, d) != LMLP_OK) return 0;
  return lin_saved_layout(d).total;
}

size_t lora_linear_workspace_bytes(const lmlp_dims* dims, int is_backward) {
  Dims d;
  if (parse_linear_dims(dims, d) != LMLP_OK) return 0;
  return is_backward ? lin_bwd_layout(d).total : lin_fwd_layout(d).total;
}

}  // extern "C"

namespace {
int linear_forward_impl(const Dims& d, const void* x, const void* w, const void* w_scales, const void* a,
                        const void* b, void* y, void* saved, size_t saved_bytes, void* workspace,
                        size_t workspace_bytes, void* stream) {
  LMLP_TRY(need_ptr(w, "w"));
  if (d.int4) LMLP_TRY(need_ptr(w_scales, "w_scales"));
  else if (w_scales) return fail(LMLP_ERR_INVALID_ARG, "w_scales must be NULL for dense weights");
  LMLP_TRY(need_ptr(a, "a"));
  LMLP_TRY(need_ptr(b, "b"));
  const LinSavedLayout SL = lin_saved_layout(d);
  const LinFwdLayout FL = lin_fwd_layout(d);
  if (d.T > 0) {
    LMLP_TRY(need_ptr(x, "x"));
    LMLP_TRY(need_ptr(y, "y"));
    LMLP_TRY(need_ptr(saved, "saved"));
    LMLP_TRY(need_ptr(workspace, "workspace"));
  }
  if (saved_bytes < SL.total) return fail(LMLP_ERR_WORKSPACE, "saved buffer smaller than lora_linear_saved_bytes()");
  if (workspace_bytes < FL.total)
    return fail(LMLP_ERR_WORKSPACE, "workspace smaller than lora_linear_workspace_bytes(dims, 0)");
  LMLP_TRY(check_device());
  if (d.T == 0) return LMLP_OK;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t T = d.T, In = d.H, Out = d.I, r = d.r, r16 = d.r16;
  const int eb = d.eb;
  float* P = reinterpret_cast<float*>(at(saved, SL.p));
  char* pT = d.bf16 ? at(saved, SL.pT) : nullptr;
  char* a_pad = at(saved, SL.a_pad);
  char* bext = at(saved, SL.bext);
  char* aext = at(workspace, FL.aext);

  PackParams pk{};
  pk.job[0] = pack_job(a_pad, In, r16, In, a, In, r, In, false);
  pk.job[1] = pack_job(bext, r16, Out, r16, b, r, Out, r, false);
  pk.job[2] = pack_job(at(saved, SL.bT), Out, r16, Out, b, r, Out, r, true);  // B^T for the backward
  pk.njobs = 3;
  LMLP_LAUNCH("pack(linear)", launch_pack(pk, eb, st));
  const void* wk = w;
  float* sc = d.q4_inkernel ? reinterpret_cast<float*>(at(workspace, FL.sc)) : nullptr;
  if (d.int4 && !d.q4_inkernel) {
    char* wq = at(workspace, FL.wq);
    LMLP_LAUNCH("dequant(W)", launch_dequant_int4(w, w_scales, Out, In, wq, st));
    wk = wq;
  }
  if (d.q4_inkernel) {
    ScalePackParams sp{};
    sp.job[0] = {static_cast<const __half*>(w_scales), sc, Out, In / 64, Out};
    sp.njobs = 1;
    LMLP_LAUNCH("pack(scales)", launch_scale_pack(sp, st));
  }

  float* rpp = reinterpret_cast<float*>(at(workspace, FL.rp_part));
  RowProjParams rp{};
  rp.T = T;
  rp.njobs = 1;
  rp.job[0] = rp_job(d, x, In, In, a_pad, In, int(r16), rpp);
  LMLP_LAUNCH("rowproj(x A^T)", launch_rowproj(rp, d.bf16, st));
  ProjFinishParams fp{};
  fp.T = T;
  fp.njobs = 1;
  fp.job[0] = fin_job(rpp, rp.job[0].kslices, T * r16, r16, int(r16), P, r16, aext, r16, d.s, pT, ld_tok(d), 0);
  LMLP_LAUNCH("finish(P)", launch_proj_finish(fp, d.bf16, st));

  GemmParams gy{};
  gy.nseg = 2;
  gy.seg[0] = seg(x, In, wk, nullptr, In, In, d.q4_inkernel, sc, nullptr);
  gy.seg[1] = seg(aext, r16, bext, nullptr, r16, r16);
  gy.M = T;
  gy.N = Out;
  gy.ldc = Out;
  gy.c0 = y;
  gy.group_m = 8;
  if (FL.nsplit > 1) {
    // split s multiplies K range [k0, k1) of x W^T (multiples of 32), the last
    // split also the adapter segment; one grouped launch, then the ordered sum
    const int S = FL.nsplit;
    float* part = reinterpret_cast<float*>(at(workspace, FL.ypart));
    GemmParams gs[8];
    const int64_t kt = (In + 31) / 32;
    for (int i = 0; i < S; ++i) {
      const int64_t k0 = kt * i / S * 32, k1 = std::min<int64_t>(kt * (i + 1) / S * 32, In);
      gs[i] = gy;
      gs[i].seg[0] = seg(static_cast<const char*>(x) + k0 * eb, In, static_cast<const char*>(wk) + k0 * eb, nullptr,
                         In, k1 - k0);
      gs[i].nseg = i == S - 1 ? 2 : 1;
      if (i != S - 1) gs[i].seg[1] = GemmSeg{};
      gs[i].c0 = part + i * T * Out;
      gs[i].tile_n = 0;
    }
    LMLP_LAUNCH("gemm(y)", launch_gemm_bf16_grouped(gs, S, 0, EPI_STORE_F32, st));
    LMLP_LAUNCH("sum(y)", launch_splitk_sum(part, S, T * Out, y, st));
    return LMLP_OK;
  }
  gy.tile_n = store_tile_n(d, T, Out);
  LMLP_LAUNCH("gemm(y)", run_gemm(gy, d, 0, EPI_STORE, st));
  return LMLP_OK;
}

// Scratch of lora_linear_forward_noalloc: one copy of this array per GPU the
// library runs on, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not the device
// address): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
constexpr size_t kNoAllocScratch = size_t(LMLP_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) char scratch[kNoAllocScratch];

int noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LMLP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(LMLP_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LMLP_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return LMLP_OK;
}
}  // namespace

extern "C" {

int lora_linear_forward(const lmlp_dims* dims, const void* x, const void* w, const void* w_scales, const void* a,
                        const void* b, void* y, void* saved, size_t saved_bytes, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Dims d;
  LMLP_TRY(parse_linear_dims(dims, d));
  return linear_forward_impl(d, x, w, w_scales, a, b, y, saved, saved_bytes, workspace, workspace_bytes, stream);
}

int lora_linear_forward_noalloc(const lmlp_dims* dims, const void* x, const void* w, const void* w_scales,
                                const void* a, const void* b, void* y, void* saved, size_t saved_bytes,
                                void* stream) {
  g_last_error.clear();
  Dims d;
  LMLP_TRY(parse_linear_dims(dims, d));
  const size_t need = lin_fwd_layout(d).total;
  if (need > kNoAllocScratch)
    return fail(LMLP_ERR_UNSUPPORTED, "workspace of these dims (" + std::to_string(need) +
                                          " bytes) exceeds the library scratch of " +
                                          std::to_string(kNoAllocScratch) + " bytes");
  LMLP_TRY(check_device());
  void* ws = nullptr;
  LMLP_TRY(noalloc_scratch(&ws));
  // nothing in the forward workspace has to start at zero: every byte a
  // kernel reads was written earlier in the same call
  return linear_forward_impl(d, x, w, w_scales, a, b, y, saved, saved_bytes, ws, kNoAllocScratch, stream);
}

int lora_linear_backward(const lmlp_dims* dims, const void* dy, const void* x, const void* w, const void* w_scales,
                         const void* a, const void* b, const void* saved, size_t saved_bytes, void* dx, void* da,
                         void* db, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Dims d;
  LMLP_TRY(parse_linear_dims(dims, d));
  LMLP_TRY(need_ptr(w, "w"));
  if (d.int4) LMLP_TRY(need_ptr(w_scales, "w_scales"));
  else if (w_scales) return fail(LMLP_ERR_INVALID_ARG, "w_scales must be NULL for dense weights");
  LMLP_TRY(need_ptr(a, "a"));
  LMLP_TRY(need_ptr(b, "b"));
  LMLP_TRY(need_ptr(da, "da"));
  LMLP_TRY(need_ptr(db, "db"));
  const LinSavedLayout SL = lin_saved_layout(d);
  const LinBwdLayout BL = lin_bwd_layout(d);
  if (d.T > 0) {
    LMLP_TRY(need_ptr(dy, "dy"));
    LMLP_TRY(need_ptr(x, "x"));
    LMLP_TRY(need_ptr(dx, "dx"));
    LMLP_TRY(need_ptr(saved, "saved"));
    LMLP_TRY(need_ptr(workspace, "workspace"));
  }
  if (saved_bytes < SL.total) return fail(LMLP_ERR_WORKSPACE, "saved buffer smaller than lora_linear_saved_bytes()");
  if (workspace_bytes < BL.total)
    return fail(LMLP_ERR_WORKSPACE, "workspace smaller than lora_linear_workspace_bytes(dims, 1)");
  LMLP_TRY(check_device());

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t T = d.T, In = d.H, Out = d.I, r = d.r, r16 = d.r16;
  const float s = d.s;
  ReduceParams rd{};
  if (T == 0) {  // no tokens: the adapter gradients are empty sums
    rd.job[0] = rd_job(nullptr, 0, 0, 0, 0, In, r, da, In, true, s, d.bf16);
    rd.job[1] = rd_job(nullptr, 0, 0, 0, 0, Out, r, db, r, false, s, d.bf16);
    rd.njobs = 2;
    LMLP_LAUNCH("reduce(zero)", launch_reduce(rd, st));
    return LMLP_OK;
  }
  const float* P = reinterpret_cast<const float*>(static_cast<const char*>(saved) + SL.p);
  const char* pT = d.bf16 ? static_cast<const char*>(saved) + SL.pT : nullptr;
  const char* a_pad = static_cast<const char*>(saved) + SL.a_pad;
  const char* bT = static_cast<const char*>(saved) + SL.bT;
  float* Q = reinterpret_cast<float*>(at(workspace, BL.q));
  char* aext = at(workspace, BL.aext);
  char* qT = d.bf16 ? at(workspace, BL.qT) : nullptr;
  float* rpa = reinterpret_cast<float*>(at(workspace, BL.rp_part));
  float* part_x = reinterpret_cast<float*>(at(workspace, BL.part_x));
  float* part_dy = reinterpret_cast<float*>(at(workspace, BL.part_dy));
  const int64_t ldT = ld_tok(d);

  const void* wk = w;
  float* scn = d.q4_inkernel ? reinterpret_cast<float*>(at(workspace, BL.scn)) : nullptr;
  if (d.q4_inkernel) {
    ScalePackParams sp{};
    sp.job[0] = {static_cast<const __half*>(w_scales), scn, Out, In / 64, sc_ld4(In), 1, 0};
    sp.njobs = 1;
    LMLP_LAUNCH("pack(scales)", launch_scale_pack(sp, st));
  } else if (d.int4) {
    char* wq = at(workspace, BL.wq);
    LMLP_LAUNCH("dequant(W)", launch_dequant_int4(w, w_scales, Out, In, wq, st));
    wk = wq;
  }
  RowProjParams rp{};
  rp.T = T;
  rp.njobs = 1;
  rp.job[0] = rp_job(d, dy, Out, Out, bT, Out, int(r16), rpa);
  LMLP_LAUNCH("rowproj(dY B)", launch_rowproj(rp, d.bf16, st));
  ProjFinishParams fp{};
  fp.T = T;
  fp.njobs = 1;
  fp.job[0] = fin_job(rpa, rp.job[0].kslices, T * r16, r16, int(r16), Q, r16, aext, r16, s, qT, ldT, 0);
  LMLP_LAUNCH("finish(Q)", launch_proj_finish(fp, d.bf16, st));

  GemmParams gx{};
  gx.nseg = 2;
  gx.seg[0] = seg(dy, Out, wk, nullptr, In, Out, d.q4_inkernel, scn, nullptr);
  gx.seg[1] = seg(aext, r16, a_pad, nullptr, In, r16);
  gx.M = T;
  gx.N = In;
  gx.ldc = In;
  gx.c0 = dx;
  gx.group_m = 8;
  gx.tile_n = store_tile_n(d, T, In);
  LMLP_LAUNCH("gemm(dX)", run_gemm(gx, d, 1, EPI_STORE, st));

  const int ntb = BL.ntb;
  ColProjParams cp{};
  cp.T = T;
  cp.job[0] = cp_job(d, x, In, In, Q, r16, qT, ldT, int(r16), part_x, ntb, BL.tr);
  cp.job[1] = cp_job(d, dy, Out, Out, P, r16, pT, ldT, int(r16), part_dy, ntb, BL.tr);
  cp.njobs = 2;
  LMLP_LAUNCH("colproj", launch_colproj(cp, d.bf16, st));
  rd.job[0] = rd_job(part_x, In * r16, ntb, r16, 0, In, r, da, In, true, s, d.bf16);
  rd.job[1] = rd_job(part_dy, Out * r16, ntb, r16, 0, Out, r, db, r, false, s, d.bf16);
  rd.njobs = 2;
  LMLP_LAUNCH("reduce", launch_reduce(rd, st));
  return LMLP_OK;
}

int lora_mlp_dequant_int4(const void* packed, const void* scales, int64_t out, int64_t in, void* w_bf16,
                          void* stream) {
  g_last_error.clear();
  if (out < 0 || in < 0) return fail(LMLP_ERR_INVALID_ARG, "negative size");
  if (in % 64) return fail(LMLP_ERR_UNSUPPORTED, "in must be a multiple of 64");
  if (out == 0 || in == 0) return LMLP_OK;
  LMLP_TRY(need_ptr(packed, "packed"));
  LMLP_TRY(need_ptr(scales, "scales"));
  LMLP_TRY(need_ptr(w_bf16, "w_bf16"));
  LMLP_TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  LMLP_LAUNCH("dequant_int4", launch_dequant_int4(packed, scales, out, in, w_bf16, st));
  return LMLP_OK;
}

int lora_mlp_mfma_probe(const void* operands, size_t operand_bytes, float* sink, int blocks, int iters,
                        void* stream) {
  g_last_error.clear();
  LMLP_TRY(need_ptr(operands, "operands"));
  LMLP_TRY(need_ptr(sink, "sink"));
  if (blocks < 1 || iters < 1) return fail(LMLP_ERR_INVALID_ARG, "blocks and iters must be >= 1");
  if (operand_bytes < size_t(blocks) * 8 * 768 * 16)
    return fail(LMLP_ERR_INVALID_ARG, "operands smaller than blocks * 8 * 768 * 16 bytes");
  LMLP_TRY(check_device());
  return hip_rc(launch_mfma_probe(operands, sink, blocks, iters, static_cast<hipStream_t>(stream)),
                "mfma probe launch");
}

int lora_mlp_profile_begin(void) {
  g_last_error.clear();
  g_prof.recs.clear();
  g_prof.used = 0;
  g_prof.on = true;
  return LMLP_OK;
}

int lora_mlp_profile_end(lmlp_kernel_time* out, int capacity, int* count) {
  g_last_error.clear();
  g_prof.on = false;
  int rc = LMLP_OK;
  int n = 0;
  // every end event: the grouped MLP records on several streams
  for (const ProfRec& r : g_prof.recs) {
    hipError_t e = hipEventSynchronize(r.e);
    if (e != hipSuccess) {
      rc = fail(LMLP_ERR_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
      break;
    }
  }
  if (rc == LMLP_OK) {
    for (const ProfRec& r : g_prof.recs) {
      if (!out || n >= capacity) break;
      float ms = 0.f;
      hipError_t e = hipEventElapsedTime(&ms, r.b, r.e);
      if (e != hipSuccess) {
        rc = fail(LMLP_ERR_HIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
        break;
      }
      std::snprintf(out[n].name, sizeof(out[n].name), "%s", r.name);
      out[n].ms = ms;
      ++n;
    }
  }
  if (count) *count = n;
  g_prof.recs.clear();
  g_prof.used = 0;
  return rc;
}

}  // extern "C"
