// Internal structures shared by the host runtime (host.cpp) and the gfx950
// kernels (kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psgd {

// Column block width of pass 2 and pass 3: 64 lanes x 4 consecutive columns.
constexpr int kColBlock = 256;
// Threads per workgroup of the streaming passes (4 wavefronts of 64).
constexpr int kThreads = 256;
// Threads per workgroup of the orthogonalization kernel.
constexpr int kOrthThreads = 512;

// One compressed matrix of the bucket (n x m, row-major inside the flat bucket).
struct TensorDesc {
  int64_t boff;   // first element of the view in the bucket
  int64_t eoff;   // first float of its error memory (multiple of 4)
  int64_t poff;   // first float of its P (n rows, row stride R; multiple of 4)
  int64_t qoff;   // first float of its Q (m rows, row stride R; multiple of 4)
  int32_t n, m;   // rows, columns
  int32_t rank;   // columns of P and Q in use (<= R); the rest are kept at zero
  int32_t vec;    // 1: m % 4 == 0 and rows start 16-byte aligned in the bucket
  int32_t view;   // index of the view in the bucket (Q draw counter word)
  int32_t rpb;    // rows per row block in pass 2 / pass 3
  int32_t nrb;    // row blocks in pass 2 / pass 3
  int32_t ncb;    // 256-column blocks in pass 2 / pass 3
  int32_t pslot;  // first partial-sum slot of pass 2 (nrb * ncb slots when nrb > 1)
  int32_t cslot;  // first arrival counter of pass 2 (ncb counters when nrb > 1)
};

// Pass 1 work item: rows [row0, row0 + nrows) of one tensor, all columns.
// Pass 2 / pass 3 work item: row block `a`, column block `b` of one tensor.
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

// Orthogonalization job: `rows` x R block at `off` (row stride R), `rank` columns.
struct OrthJob {
  int64_t off;
  int32_t rows;
  int32_t rank;
};

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
  float inv_scale;
  int32_t* found_inf;
};

struct Pass2Args {
  const Tile* tiles;
  int32_t ntiles;
  const TensorDesc* td;
  const void* bucket;
  const float* E;
  const float* P;
  float* Q;
  float* partial;
  int32_t* counters;
  float inv_scale;
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
  const float* Q;
  float inv_scale;
  const int32_t* found_inf;
};

// Launchers (kernels.hip). R is the padded rank (1, 2, 4, 8, 16 or 32).
hipError_t launch_pass1(int R, int rows_per_lane, bool f16, bool ef, const Pass1Args& a,
                        hipStream_t s);
hipError_t launch_pass2(int R, bool f16, bool ef, const Pass2Args& a, hipStream_t s);
hipError_t launch_pass3(int R, bool f16, bool ef, const Pass3Args& a, hipStream_t s);
hipError_t launch_orth(int R, const OrthJob* jobs, int njobs, float* base, double eps,
                       const int32_t* found_inf, hipStream_t s);
hipError_t launch_qinit(int R, const QInitJob* jobs, int njobs, int64_t max_count,
                        float* Q, uint64_t seed, uint64_t bucket_key, uint64_t epoch,
                        hipStream_t s);
hipError_t launch_unscale_only(const FlatTile* ftiles, int nftiles, void* bucket,
                               float inv_scale, int32_t* found_inf, bool check,
                               hipStream_t s);

// Rows of one pass-1 row group per wavefront, as chosen for a padded rank R.
int pass1_rows_per_lane(int R);

}  // namespace psgd
