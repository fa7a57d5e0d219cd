// Launch parameters and launchers of the gfx950 kernels (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <functional>

namespace lmlp {

// EPI_STORE_F32: the fp32 accumulators themselves (a split-K partial), no rounding.
enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_STORE_F32 = 3 };

// One K segment of a GEMM: C += A[:, seg] * B[seg, :].
struct GemmSeg {
  const void* a;    // [M][lda], K contiguous, compute dtype
  const void* b0;   // NT: [N][ldb] K contiguous; NN: [K][ldb] N contiguous
  const void* b1;   // gate/up product only: the up-projection rows (b0 = gate)
  const void* bs0;  // 4-bit B only: fp16 scales of b0 (one per 64 codes)
  const void* bs1;  // 4-bit B only: scales of b1
  int64_t lda;      // elements
  int64_t ldb;      // elements (for 4-bit B: codes per row)
  int64_t K;        // contraction length (elements), multiple of the 16-byte chunk
  int32_t bint4;    // B stored as 4-bit blocks
  int32_t pad_;
};

struct GemmParams {
  GemmSeg seg[3];
  int32_t nseg;
  int32_t group_m;  // tiles of M visited before moving along N (L2 reuse)
  int32_t tiles_m, tiles_n;
  int64_t M, N;     // output rows, columns (gate/up: N = I, pairs of columns)
  int64_t ldc;      // row stride of every output / saved activation
  void* c0;         // STORE: C. SWIGLU_FWD: G. SWIGLU_BWD: dG
  void* c1;         // SWIGLU_FWD: U. SWIGLU_BWD: dU
  void* c2;         // Z (forward: input of the down product; backward: optional)
  const void* g_in; // SWIGLU_BWD: saved G
  const void* u_in; // SWIGLU_BWD: saved U
  // SWIGLU_BWD, optional (bf16 kernel, pj_part0 != nullptr, pj_r16 = 16): the
  // epilogue also forms the rank-16 products of dG, dU and Z (Z is then not
  // written):
  //  * row products dG B_g (into pj_part0) and dU B_u (pj_part1), one split-K
  //    slice per tile column: fp32 [slices][pj_T][16], pj_T = tokens, slice
  //    pj_slice0 + n0 / tile width;
  //    pj_b0 / pj_b1 = B_g^T / B_u^T as bf16 [16][pj_ldb];
  //  * column products P_g^T dG, P_u^T dU, Q_d^T Z (into pj_cdg, pj_cdu, pj_cz),
  //    one slice per 256-row tile: fp32 [tiles_m][pj_ncol][16] (column-major in
  //    the rank); pj_pguT = [P_g^T; P_u^T] as bf16 [32][pj_ldt], pj_qdT = Q_d^T
  //    as bf16 [16][pj_ldt], zero past T.
  const void* pj_b0;
  const void* pj_b1;
  float* pj_part0;
  float* pj_part1;
  int64_t pj_ldb, pj_T;
  int32_t pj_r16;
  const void* pj_pguT;
  const void* pj_qdT;
  int64_t pj_ldt;
  float* pj_cdg;
  float* pj_cdu;
  float* pj_cz;
  int64_t pj_ncol;    // row stride (columns) of the column-product partials
  int32_t pj_slice0;  // first row-product slice of this launch
  // STORE and SWIGLU_BWD: tile width, 256 (0 = default) or 128 (SWIGLU_BWD:
  // row-product slices are then per 128 columns)
  int32_t tile_n;
};

// Up to kMaxGemmGroups products of one kind (same NN / epilogue / tile
// width) in one launch; set by the grouped launcher.
constexpr int kMaxGemmGroups = 8;
struct GemmGroups {
  GemmParams p[kMaxGemmGroups];
  int32_t start[kMaxGemmGroups + 1];  // first workgroup of each group (multiples of 8), then the total
  int32_t n;
};

// fp32 products (register-staged general kernel)
hipError_t launch_gemm_f32(const GemmParams& p, int nn, int epi, hipStream_t stream);
// dense bf16 operands only (LDS-DMA staging); needs every row stride * 256 < 2^31 bytes
hipError_t launch_gemm_bf16(const GemmParams& p, int nn, int epi, hipStream_t stream);
// The same products, n of them of one kind (grouped MLP experts), in
// launches of up to kMaxGemmGroups products each.
hipError_t launch_gemm_bf16_grouped(const GemmParams* ps, int n, int nn, int epi, hipStream_t stream);
// Tables of several launches staged together (one read of the pinned ring
// for all of them): add() copies a table into the batch and returns the
// device address it will have (nullptr: no room left; make_room() then
// enqueues what the batch holds so far); defer() queues a launch that reads
// such a table, to go out, in order, once the batch is staged.
struct TableBatch {
  virtual ~TableBatch() = default;
  virtual void* add(const void* src, size_t bytes) = 0;
  virtual hipError_t make_room() = 0;
  virtual void defer(std::function<hipError_t()> launch) = 0;
};

// The same with the parameter blocks in device memory: `table` (device, at
// least n * sizeof(GemmParams) bytes, 16-byte aligned) receives the n blocks
// on `stream` (through the pinned ring, or small copy kernels), and one
// launch per kMaxTableGroups products reads them there. With `batch`, the
// blocks go into the batch instead (`table` unused) and the launches are
// deferred to it.
constexpr int kMaxTableGroups = 512;
hipError_t launch_gemm_bf16_grouped_table(const GemmParams* ps, int n, int nn, int epi, GemmParams* table,
                                          hipStream_t stream, TableBatch* batch = nullptr);
// Products whose leading K segments have a 4-bit B operand (seg.bint4), on
// the eight-wave kernel: NT (gate/up, down): codes [N][K/2] bytes (ldb = K),
// scales fp32 block-major [K/64][N] (bs0/bs1); NN (dZ, dX): codes [K][N/2]
// bytes (ldb = N), scales fp32 row-major [K][ld_sc] with ld_sc =
// roundup(N/64, 4) (bs0). K and N multiples of 64; the segments after the
// 4-bit ones are dense bf16.
hipError_t launch_gemm_bf16_q4(const GemmParams& p, int nn, int epi, hipStream_t stream);


// Row projection, split along K: part[ks][t][n] = sum over k in slice ks of
// X[t][k] * W[n][k] (slice ks = [ks*kb, (ks+1)*kb)), for up to two jobs per
// launch. launch_proj_finish sums the slices.
struct RowProjJob {
  const void* x;    // [T][ldx]
  const void* w;    // [n1p][ldw], K contiguous, zero rows past the real rank
  float* part;      // [kslices][T][n1p]
  int64_t ldx, ldw, K;
  int64_t kb;       // elements per slice, a multiple of four MFMA k-steps
  int32_t n1p;      // multiple of 16
  int32_t kslices;
  int64_t T;        // token rows of this job (0: the launch's T)
};
// job capacities: every parameter block stays under 3.8 KB of kernel arguments
// (table: when set, the launch's njobs jobs are read from this device array
// instead of job[], so that one launch can carry more jobs than the kernel
// arguments hold; the launcher then takes the same jobs on the host as
// `hjobs`, with every T filled in, to size the grid.)
struct RowProjParams {
  RowProjJob job[52];
  int32_t njobs;
  int32_t nsl;      // set by the launcher: 64-column slices of the widest job
  int64_t T;
  const RowProjJob* table;
};
hipError_t launch_rowproj(const RowProjParams& p, int dtype_bf16, hipStream_t stream,
                          const RowProjJob* hjobs = nullptr);

// v(t, n) = sum_k part[k][t][n] (k < nparts, in order), n < n1p; written as
// out_f32[t][col_off + n] (fp32), out_c[t][col_off + n] = scale * v (compute
// dtype) and outT[col_off + n][t] (compute dtype, zero for T <= t < ldT);
// each output optional. A saved fp32 matrix with nparts = 1 gives its
// transposed copy.
struct ProjFinishJob {
  const float* part;
  int64_t part_stride;  // elements between partials
  int64_t ld_part;      // row stride of a partial (elements)
  float* out_f32;
  int64_t ld_f32;
  void* out_c;
  int64_t ld_c;
  void* outT;
  int64_t ldT;          // multiple of 64
  float scale;
  int32_t nparts;
  int32_t n1p;          // multiple of 4
  int32_t col_off;
  int64_t T;            // token rows of this job (0: the launch's T)
};
struct ProjFinishParams {
  ProjFinishJob job[36];
  int32_t njobs;
  int32_t tall;  // set by the launcher: narrow jobs in up to 64-token tiles
  int64_t T;
  const ProjFinishJob* table;
};
hipError_t launch_proj_finish(const ProjFinishParams& p, int dtype_bf16, hipStream_t stream,
                              const ProjFinishJob* hjobs = nullptr);

// Column projection: part[tb][k][n] = sum_{t in block tb} X[t][k] * P[t][n]
// (fp32 partials over token blocks; reduced by launch_reduce). bf16 reads the
// transposed P (pT, compute dtype, token-contiguous, zero past T) and covers
// 256 features x 128 columns per workgroup; fp32 reads P and covers 64 x 64.
struct ColProjJob {
  const void* x;    // [T][ldx]
  const float* p;   // fp32 path: [T][ldp]
  const void* pT;   // bf16 path: [n2p][ldpT]
  float* part;      // [ntb][K][n2p]
  int64_t ldx, ldp, ldpT, K;
  int64_t tr;       // tokens per block (multiple of 32)
  int32_t n2p;      // multiple of 16, <= 512
  int32_t ntb;      // token blocks
  int32_t kblocks;  // feature blocks (256 bf16, 64 fp32)
  int32_t nchunks;  // column chunks (128 bf16, 64 fp32)
  int64_t T;        // tokens of this job (0: the launch's T)
};
struct ColProjParams {
  ColProjJob job[38];
  int32_t njobs;
  int32_t pad_;
  int64_t T;
  const ColProjJob* table;
};
hipError_t launch_colproj(const ColProjParams& p, int dtype_bf16, hipStream_t stream,
                          const ColProjJob* hjobs = nullptr);

// Fixed-order sum of partials into a final, scaled, optionally transposed
// matrix in fp32 or bf16: dst(i, j) = scale * sum_c src[c][i][col_off + j].
struct ReduceJob {
  const float* src;
  void* dst;
  int64_t chunk_stride, ld_src, rows, cols, ld_dst;
  float scale;
  int32_t nchunk;
  int32_t col_off;
  int32_t transpose;  // write dst[j][i]
  int32_t dst_bf16;
  int32_t pad_;
};
struct ReduceParams {
  ReduceJob job[46];
  int32_t njobs;
  int32_t tall;  // set by the launcher: rank-wide jobs in 64-row tiles
  const ReduceJob* table;
};
hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream, const ReduceJob* hjobs = nullptr);

// Zero-padded copy of an adapter factor into a GEMM/projection operand
// layout: dst[i][j] = src(i, j) (or src(j, i) if transpose) inside the source
// extent, 0 elsewhere, for i < rows, j < cols.
struct PackJob {
  void* dst;
  const void* src;  // null: fill zeros
  int64_t ld_dst, rows, cols;
  int64_t ld_src, srows, scols;
  int32_t transpose;
  int32_t pad_;
};
struct PackParams {
  PackJob job[52];
  int32_t njobs;
  int32_t pad_;
  const PackJob* table;
};
hipError_t launch_pack(const PackParams& p, int elem_bytes, hipStream_t stream, const PackJob* hjobs = nullptr);

// fp16 block scales [rows][nb] -> fp32 [nb][ld_dst]
// fp16 block scales [rows][nb] -> fp32: block-major dst[b][r] (row_major 0,
// the NT products' layout) or row-major dst[r][b] (row_major 1, the NN
// products'); ld_dst is the destination row stride in elements
struct ScalePackJob {
  const __half* src;
  float* dst;
  int64_t rows, nb, ld_dst;
  int32_t row_major;
  int32_t pad_;
};
struct ScalePackParams {
  ScalePackJob job[3];
  int32_t njobs;
  int32_t pad_;
};
hipError_t launch_scale_pack(const ScalePackParams& p, hipStream_t stream);

// bf16 matrix-core ceiling: blocks x 8 waves x iters x 32 MFMA 16x16x32 on
// operands read once from `ops` (blocks * 8 * 768 uint4)
hipError_t launch_mfma_probe(const void* ops, float* sink, int blocks, int iters, hipStream_t stream);

// Copy `bytes` of host data to the device array `dst` on `stream`, ordered
// with the stream's other work: through a pinned host ring, read by one
// workgroup on the stream, when it can, else with copy kernels that carry the
// data in their arguments (under stream capture, or while a read from the
// ring region it would reuse has not run yet). The host never waits.
hipError_t stage_device_table(const void* src, size_t bytes, void* dst, hipStream_t stream);

// Split-K finish: y[i] = bf16_rne(part[0][i] + part[1][i] + ... + part[nsplit-1][i]),
// summed in that order; part holds nsplit slices of n fp32 values (n a multiple of 4).
hipError_t launch_splitk_sum(const float* part, int nsplit, int64_t n, void* y_bf16, hipStream_t stream);

// 4-bit block weight -> bf16 (same decode as the GEMM loaders).
hipError_t launch_dequant_int4(const void* packed, const void* scales, int64_t out, int64_t in,
                               void* w_bf16, hipStream_t stream);

// RMSNorm of token rows [T][H] with a frozen weight gamma [H] (all in the
// compute dtype; rstd fp32 [T]):
//   NORM_FWD    xn = x * rstd * gamma, rstd written
//   NORM_APPLY  xn from the given rstd
//   NORM_BWD    dx = rstd * (gamma g - xhat * mean(gamma g xhat)), xhat = x rstd;
//               g may be the same buffer as dx
enum { NORM_FWD = 0, NORM_APPLY = 1, NORM_BWD = 2 };
struct NormParams {
  const void* x;
  const void* gamma;
  void* xn;
  float* rstd;
  const void* g;
  void* dx;
  int64_t T, H;  // H a multiple of the 16-byte chunk
  float eps;
  int32_t mode;
};
hipError_t launch_rmsnorm(const NormParams& p, int dtype_bf16, hipStream_t stream);

}  // namespace lmlp
