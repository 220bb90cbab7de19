// Internal structures shared by the host runtime (host.cpp) and the gfx950
// kernels (kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "powersgd.h"

namespace psgd {

// Column block width of pass 2 and pass 3: 64 lanes x 4 consecutive columns.
constexpr int kColBlock = 256;
// Threads per workgroup of the streaming passes (4 wavefronts of 64).
constexpr int kThreads = 256;

// One compressed matrix of the bucket (n x m, row-major inside the flat bucket).
//
// Pass 1 work items are row blocks of rpb1 full rows: the 256 threads of a
// workgroup form 256 / lprw row slots of lprw threads, a thread owning 4 consecutive
// columns per sweep of 4 * lprw columns, so every dot product stays inside one
// workgroup. Pass 2 work items are (row block of rpb rows) x (256-column block), pass
// 3 ones (row block of rpb3 rows) x (256-column block): a wavefront's 64 lanes form
// 64 / lpr row slots of lpr lanes, a lane owning 4 consecutive columns. Pass 2 writes
// one partial Q per row block when nrb > 1; a separate reduction sums them.
struct TensorDesc {
  int64_t boff;   // first element of the view in the bucket
  int64_t eoff;   // first float of its error memory (multiple of 4)
  int64_t poff;   // first float of its P (n rows, row stride R; multiple of 4)
  int64_t qoff;   // first float of its Q (m rows, row stride R; multiple of 4)
  int32_t n, m;   // rows, columns
  int32_t rank;   // columns of P and Q in use (<= R); the rest are kept at zero
  int32_t vec;    // 1: m % 4 == 0 and rows start 16-byte aligned in the bucket
  int32_t view;   // index of the view in the bucket (Q draw counter word)
  int64_t goff;   // first double of its P Gram partials (one per pass-1 row block)
  int64_t qtoff;  // matrix-core ranks: first float of Q^T (R rows of mstride floats)
  int32_t mstride;  // row stride of Q^T: m rounded up to a multiple of 4 (padding zero)
  int32_t rpb3;     // pass 3: rows per row block (its own tiling, same lane geometry)
  int32_t lprw;   // pass 1: threads per row slot (power of two, <= 256)
  int32_t rpb1;   // pass 1: rows per row block
  int32_t lpr;    // pass 2/3: lanes per row slot (power of two, <= 64)
  int32_t rpb;    // pass 2/3: rows per row block
  int32_t nrb;    // pass 2/3: row blocks
  int32_t ncb;    // pass 2/3: 256-column blocks
  int32_t pslot;  // first pass-2 partial slot (nrb * ncb slots when nrb > 1)
  int32_t ncg1;   // matrix-core ranks: pass-1 column groups of kPass1Cols columns
  int64_t p1off;  // matrix-core ranks: first float of its pass-1 partial P (ncg1 x n x R)
};

// Work item of the streaming passes: row block `a` (and column block `b` in
// passes 2 and 3) of a tensor.
struct Tile {
  int32_t tensor;
  int32_t a;
  int32_t b;
  int32_t pad;
};

// A contiguous element range of an uncompressed view (fp16 check / unscale).
struct FlatTile {
  int64_t start;
  int64_t len;
};

// Orthogonalization job: the `rows` x R block at `off` (row stride R, `rank` columns in
// use). Its Gram matrix arrives as `nparts` partials of R(R+1)/2 doubles at `goff`
// (packed upper triangle), partial p covering rows [p * rpp, (p + 1) * rpp).
struct OrthJob {
  int64_t off;
  int64_t goff;
  int64_t toff;     // >= 0: also write the result transposed (R rows of tstride floats)
  int32_t rows;
  int32_t rank;
  int32_t nparts;
  int32_t rpp;
  int32_t tstride;
  int32_t ncg;      // > 0: the rows are the sum of ncg partials at part (group-major,
                    // rows x R each), which the Gram kernel adds and writes to off
  int64_t part;
};

// Packed upper-triangle index of Gram entry (i, j), i <= j < R.
__host__ __device__ constexpr int tri_index(int i, int j, int R) {
  return i * R - i * (i - 1) / 2 + (j - i);
}
template <int R> constexpr int gram_size() { return R * (R + 1) / 2; }

// Initial-Q job: the m x rank draw of one view, stored with row stride R.
struct QInitJob {
  int64_t qoff;
  int32_t m;
  int32_t rank;
  int32_t view;
  int32_t pad;
};

struct Pass1Args {
  const Tile* tiles;
  int32_t ntiles;
  const FlatTile* ftiles;  // fp16 only: inf/NaN check of uncompressed views
  int32_t nftiles;
  const TensorDesc* td;
  void* bucket;
  float* E;
  const float* Q;
  float* P;
  // matrix-core ranks: P of each (row block, column group) work item, a partial sum
  // over the group's columns, at p1off + (group * n + row) * R
  float* Ppart;
  // With error feedback E's place keeps M' of the previous step (binary32 in E, or 16
  // bits in Eh); its error is rebuilt as E = M'_prev - Pe Q^T (with pass 3's rounding)
  // with Pe the previous orthogonalized P (Q being the warm-start Q). Null when E's
  // place holds the error itself (first call, after an import, without warm start).
  const float* Pe;
  // With Pe: device flag, non-zero while E's place still holds the error itself (then
  // nothing is rebuilt); pass 3 of a step that ran clears it.
  const int32_t* wflag;
  // E's place double-buffered (an fp16 bucket's M'): two places wstride floats apart,
  // *widx (0 or 1) naming the current one (M'_prev or the error); pass 1 writes M' into
  // the other. wstride 0: one place, read and overwritten in place (widx unused).
  const int32_t* widx;
  int64_t wstride;
  const float* QT;         // matrix-core ranks: Q^T (B fragments as 16-byte loads)
  double* gram;            // P Gram partials (ranks <= 8: computed here)
  uint16_t* Eh;            // 16-bit state: E's place (E's offsets)
  uint16_t* Mh;            // 16-bit state: M' written here (E's offsets; Eh itself with
                           // error feedback)
  float inv_scale;
  int32_t* found_inf;
};

struct Pass2Args {
  const Tile* tiles;
  int32_t ntiles;
  const TensorDesc* td;
  const void* bucket;
  const float* E;
  const float* P;          // vector ranks: P as pass 1 left it; matrix-core: orthogonalized
  float* Pout;             // vector ranks: orthogonalized P (written by column block 0 tiles)
  const double* gram;      // vector ranks: the Gram partials of P from pass 1
  double eps;              // vector ranks: orthogonalization epsilon
  float* Q;
  float* QT;               // matrix-core ranks: Q^T, written next to Q (else null)
  float* partial;
  const uint16_t* Mh;      // 16-bit state: M' (E's offsets; E's place with error feedback)
  float inv_scale;
  const int32_t* found_inf;
  const int32_t* widx;     // E's places as in Pass1Args; M' is read from the one pass 1
  int64_t wstride;         // wrote
};

// Sum of pass-2 partial slots: one work item per (tensor, column block).
struct Pass2ReduceArgs {
  const Tile* tiles;       // a = unused, b = column block
  int32_t ntiles;
  const TensorDesc* td;
  const float* partial;
  float* Q;
  float* QT;               // matrix-core ranks: Q^T, written next to Q (else null)
  const int32_t* found_inf;
};

struct Pass3Args {
  const Tile* tiles;
  int32_t ntiles;
  const FlatTile* ftiles;  // fp16 only: unscale of uncompressed views
  int32_t nftiles;
  const TensorDesc* td;
  void* bucket;
  float* E;
  const float* P;
  float* Q;                // vector ranks: written here for tensors split into row blocks
  const float* partial;    // vector ranks: pass-2 partial slots (summed here)
  uint16_t* Eh;            // 16-bit state: E's place (E's offsets)
  const uint16_t* Mh;      // 16-bit state: M' (E's offsets; Eh itself with error feedback)
  float inv_scale;
  const int32_t* found_inf;
  // error materialization: E = M' - P Q^T written here as binary32 (E's offsets); with
  // Eout null it goes back into E's current place (in 16 bits into Eh for a 16-bit
  // state)
  float* Eout;
  // Buckets keeping M' in E's place: the device flag that says E's place still holds the
  // error itself. Pass 3 of a step that ran clears it; the materialization reads it (set:
  // the error is copied as it is). Null: E's place holds M'.
  int32_t* wflag;
  // E's places as in Pass1Args: pass 3 of a step that ran makes the place pass 1 wrote
  // the current one; the materialization reads the current one.
  int32_t* widx;
  int64_t wstride;
};

// Precision of the state a bucket keeps: kStF32 for the hook on fp32 or fp16 buckets;
// kStF16 / kStBF16 for the hook wrapped by fp16_compress_wrapper / bf16_compress_wrapper
// (the bucket stays fp32; M', E, P, Q and M_hat hold 16-bit values, rounded to nearest
// even where each is formed; P and Q keep fp32 containers).
constexpr int kStF32 = 0;
constexpr int kStF16 = 1;
constexpr int kStBF16 = 2;

// Launchers (kernels.hip). R is the padded rank (1, 2, 4, 8, 16 or 32); st the state
// precision (a 16-bit state needs an fp32 bucket).
hipError_t launch_pass1(int R, bool f16, bool ef, int st, const Pass1Args& a, hipStream_t s);
// wide_only (16-bit state, vector ranks): every tensor of the table has 16-byte aligned
// rows at least 256 columns wide, so a kernel compiled with that access mode alone can
// run (fewer registers, more wavefronts in flight for the state's 8-byte accesses).
hipError_t launch_pass2(int R, bool f16, bool ef, int st, bool wide_only, const Pass2Args& a,
                        hipStream_t s);
hipError_t launch_pass2_reduce(int R, int st, const Pass2ReduceArgs& a, hipStream_t s);
hipError_t launch_pass3(int R, bool f16, bool ef, int st, const Pass3Args& a, hipStream_t s);
// A state with error feedback (precision st): the error E = M' - P Q^T of every tensor,
// from the M' kept in E's current place (in a.E, or a.Mh = a.Eh for a 16-bit state) and
// the step's P and Q, into a.Eout (binary32, E's layout) or, with a.Eout null, back into
// E's current place, with pass 3's tiling and arithmetic, so the values are the ones
// pass 3's M_hat implies.
hipError_t launch_error_materialize(int R, int st, const Pass3Args& a, hipStream_t s);
// *flag = value (one thread; no memset node, so it can sit in a captured graph).
hipError_t launch_set_flag(int32_t* flag, int32_t value, hipStream_t s);
// Double-double Gram partials of each job's rows (one work item per kGramRows rows).
// Jobs with ncg > 0 first form their rows as the sum of the pass-1 partials at part
// (in group order, rounded to the state's precision st) and write them to base.
hipError_t launch_gram(int R, const Tile* tiles, int ntiles, const OrthJob* jobs,
                       float* base, const float* part, double* gram,
                       const int32_t* found_inf, int st, hipStream_t s);
// Gram-Schmidt of each job's block from its double-double Gram partials: the r x r
// transforms (tmat: R x R fp64 per job) in one launch, then X <- X T.
hipError_t launch_orth(int R, const OrthJob* jobs, int njobs, int max_rows, float* base,
                       float* tbase, const double* gram, double* tmat, double eps,
                       const int32_t* found_inf, int st, hipStream_t s);
hipError_t launch_qinit(int R, const QInitJob* jobs, int njobs, int64_t max_count,
                        float* Q, uint64_t seed, uint64_t bucket_key, uint64_t epoch, int st,
                        hipStream_t s);
// The raw m x rank draw of one view (row stride rank) and, when words is not null, its
// Philox output words (4 per counter block).
hipError_t launch_qdraw(int64_t m, int rank, int view, float* out, uint64_t* words,
                        uint64_t seed, uint64_t bucket_key, uint64_t epoch, hipStream_t s);
// 16-bit state outside the compressed views: x <- x rounded to st's precision, in place
// over fp32 ranges (the wrapper's cast and cast back).
hipError_t launch_round_only(const FlatTile* ftiles, int nftiles, void* bucket, int st,
                             hipStream_t s);
// dst[i] = the 16-bit state value src[i] as fp32, i < count (introspection of E).
hipError_t launch_widen16(const uint16_t* src, float* dst, int64_t count, int st, hipStream_t s);
// Zeroes elements [start, start + count) of a fp32 or fp16 buffer (a fill kernel, so
// the call can be captured in a graph).
hipError_t launch_fill_zero(void* base, bool f16, int64_t start, int64_t count, hipStream_t s);
hipError_t launch_unscale_only(const FlatTile* ftiles, int nftiles, void* bucket,
                               float inv_scale, int32_t* found_inf, bool check,
                               hipStream_t s);

// Tuning constants of the vector-rank streaming passes (overridable at build time).
#ifndef PSGD_PASS1_ROWS
#define PSGD_PASS1_ROWS 4  // pass 1 rows in flight per thread, padded ranks <= 4
#endif
#ifndef PSGD_PASS2_ROWS
#define PSGD_PASS2_ROWS 8  // pass 2 rows in flight per lane, padded ranks <= 4
#endif
#ifndef PSGD_PASS3_ROWS
#define PSGD_PASS3_ROWS 8  // pass 3 rows in flight per lane, padded ranks <= 8
#endif
// Rows in flight for a 16-bit state (its M' and E accesses are 8 bytes per lane).
#ifndef PSGD_PASS1_ROWS_H
#define PSGD_PASS1_ROWS_H PSGD_PASS1_ROWS
#endif
#ifndef PSGD_PASS2_ROWS_H
#define PSGD_PASS2_ROWS_H PSGD_PASS2_ROWS
#endif
#ifndef PSGD_PASS3_ROWS_H
#define PSGD_PASS3_ROWS_H PSGD_PASS3_ROWS
#endif
#ifndef PSGD_TILES_PER_BUCKET
#define PSGD_TILES_PER_BUCKET 16384  // work items aimed at per pass (before clamping)
#endif
#ifndef PSGD_PASS2_TILE_SCALE
#define PSGD_PASS2_TILE_SCALE 4  // pass-2 work items this many times larger (vector ranks)
#endif
#ifndef PSGD_PASS3_TILE_SCALE
#define PSGD_PASS3_TILE_SCALE 4  // pass-3 work items this many times taller (vector ranks)
#endif

// Rows loaded per thread before use in pass 1 (P = M' Q), by padded rank.
constexpr int pass1_unroll(int R) { return R <= 4 ? PSGD_PASS1_ROWS : 1; }
// Pass 1 row sums parked in LDS per workgroup when a row slot spans several
// wavefronts (rows of the tile x wavefronts per slot); the plan keeps tiles within it.
constexpr int kPass1SlotSums = 544;
// Pass 1 also accumulates the Gram partials of P up to this padded rank; above it a
// separate Gram kernel reads P.
constexpr int kMaxFusedGramRank = 8;
// Padded ranks from this value up run the three passes on matrix cores
// (v_mfma_f32_16x16x4f32): pass-1 row blocks are 32 rows, two MFMA row groups of 16
// (the four wavefronts split the columns, and each Q^T fragment serves both groups),
// pass 2 tiles are kMfmaPass2Rows and pass 3 tiles kMfmaRowBlock rows x 256 columns
// (64 per wavefront).
constexpr int kMfmaMinRank = 16;
constexpr int kMfmaPass1Rows = 32;
// Matrix-core pass 1 splits rows into groups of this many columns (the work items of a
// row block run side by side, so the running workgroups read neighbouring rows); each
// writes a partial P, summed in the Gram kernel.
constexpr int kPass1Cols = 4096;
constexpr int kMfmaRowBlock = 1024;
// Matrix-core pass 2 row blocks: twice the pass-3 ones, half the Q partial slots to
// write and to sum.
constexpr int kMfmaPass2Rows = 2048;
// Threads per workgroup of the pass-2 partial reduction.
constexpr int kReduceThreads = 1024;
// Vector ranks: floats of orthogonalized P rows a pass-2 workgroup keeps in LDS (the
// plan keeps row blocks at or below kPass2StageFloats / R rows).
constexpr int kPass2StageFloats = 4096;
// Largest row or column count of a compressed matrix. The kernels index rows and
// columns in 32 bits and address up to a few thousand rows past a work item's last row
// before clamping (rows in flight times row slots), so the limit keeps that headroom.
constexpr int64_t kMaxMatrixDim = 2147483647LL - 65536;
// Rows per Gram partial of the separate Gram kernel.
constexpr int kGramRows = 256;
// Rows transformed by one workgroup of the orthogonalization kernel, by padded rank
// (matrix-core ranks: a row per thread).
constexpr int kOrthRows = 1024;
constexpr int orth_rows(int R) { return R >= kMfmaMinRank ? kThreads : kOrthRows; }
// Threads of the workgroup that computes one matrix's transform T (a thread per element
// of the 32 x 32 factor in the recurrence).
constexpr int kOrthThreads = 1024;

// One n x m matrix as the bucket plan lays out a bucket that holds only that matrix
// (every buffer offset is 0; compressed without the rate test at rank min(r, n, m)):
// its descriptor, its orthogonalization and draw jobs, the work-item counts of each
// pass and the sizes of the working buffers. Host only (host.cpp).
struct MatrixLayout {
  TensorDesc d;
  int R;                                      // padded rank
  OrthJob pjob, qjob;                         // Gram-Schmidt of P and of the draw of Q
  QInitJob qinit;
  int32_t ntiles1, ntiles2, ntiles3, ntiles2r, npgram, nqgram;
  int32_t nrb3;                               // pass-3 row blocks
  int64_t p_floats, q_floats, qt_floats, partial_floats, gram_doubles, ppart_floats;
};
powersgd_status matrix_layout(const powersgd_hparams& hp, int64_t n, int64_t m,
                              MatrixLayout& out);

// Records `msg` as the calling thread's powersgd_last_error detail and returns s.
powersgd_status report_error(powersgd_status s, const char* msg);

}  // namespace psgd
