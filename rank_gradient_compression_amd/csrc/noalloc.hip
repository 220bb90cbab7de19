// powersgd_compress_matrix_noalloc: one PowerSGD compression step of one matrix
// ("DDP Communication Hooks -- PyTorch 1.11.0", section "PowerSGD Hooks",
// powerSGD_hook steps 3.1 to 3.7 for a single tensor, with error feedback) that
// allocates nothing. The matrix is laid out exactly as the bucket plan lays out a
// bucket holding only it, and the same kernels run on it; every working buffer (work
// items, padded factors, Gram partials, transforms, partial sums) lives in one fixed
// device array instead of allocated state. The work-item tables are written by a
// kernel from launch arguments, so a call enqueues kernel launches only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "internal.h"

namespace psgd {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

// The working memory of powersgd_compress_matrix_noalloc; every device holds its own
// copy. Host code reaches it only through the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's working array, looked up once per device.
hipError_t scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

// Where each table and buffer sits in the working array.
struct Carve {
  TensorDesc* desc;
  OrthJob* pjob;
  OrthJob* qjob;
  QInitJob* qinit;
  Tile *tiles1, *tiles2, *tiles3, *tiles2r, *pgram, *qgram;
  float *P, *Praw, *Ppart, *Q, *QT, *partial;
  double *gram, *tmat;
  size_t bytes;
};

Carve carve(unsigned char* base, const MatrixLayout& L) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = base + off;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  Carve c{};
  c.desc = reinterpret_cast<TensorDesc*>(take(sizeof(TensorDesc)));
  c.pjob = reinterpret_cast<OrthJob*>(take(sizeof(OrthJob)));
  c.qjob = reinterpret_cast<OrthJob*>(take(sizeof(OrthJob)));
  c.qinit = reinterpret_cast<QInitJob*>(take(sizeof(QInitJob)));
  c.tiles1 = reinterpret_cast<Tile*>(take(sizeof(Tile) * L.ntiles1));
  c.tiles2 = reinterpret_cast<Tile*>(take(sizeof(Tile) * L.ntiles2));
  c.tiles3 = reinterpret_cast<Tile*>(take(sizeof(Tile) * L.ntiles3));
  c.tiles2r = reinterpret_cast<Tile*>(take(sizeof(Tile) * L.ntiles2r));
  c.pgram = reinterpret_cast<Tile*>(take(sizeof(Tile) * L.npgram));
  c.qgram = reinterpret_cast<Tile*>(take(sizeof(Tile) * L.nqgram));
  c.P = reinterpret_cast<float*>(take(sizeof(float) * L.p_floats));
  c.Praw = reinterpret_cast<float*>(
      take(L.R <= kMaxFusedGramRank ? sizeof(float) * L.p_floats : 0));
  c.Ppart = reinterpret_cast<float*>(take(sizeof(float) * L.ppart_floats));
  c.Q = reinterpret_cast<float*>(take(sizeof(float) * L.q_floats));
  c.QT = reinterpret_cast<float*>(take(sizeof(float) * L.qt_floats));
  c.partial = reinterpret_cast<float*>(take(sizeof(float) * L.partial_floats));
  c.gram = reinterpret_cast<double*>(take(sizeof(double) * L.gram_doubles));
  c.tmat = reinterpret_cast<double*>(take(sizeof(double) * L.R * L.R));
  c.bytes = off;
  if (L.R > kMaxFusedGramRank) c.Praw = nullptr;
  if (L.qt_floats == 0) c.QT = nullptr;
  return c;
}

// The tables of the one matrix, in the bucket plan's order: pass 1 row blocks; pass 2
// and pass 3 (row block, column block) per column block; the column blocks whose
// row-block partials are summed; the Gram-kernel chunks of P and of Q.
struct SetupArgs {
  TensorDesc d;
  OrthJob pjob, qjob;
  QInitJob qinit;
  int32_t ntiles1, ntiles2, ntiles3, ntiles2r, npgram, nqgram, nrb3;
  Carve c;
};

__global__ void __launch_bounds__(256) k_noalloc_setup(SetupArgs a) {
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  if (i0 == 0) {
    *a.c.desc = a.d;
    *a.c.pjob = a.pjob;
    *a.c.qjob = a.qjob;
    *a.c.qinit = a.qinit;
  }
  const int32_t nrb = a.d.nrb;
  const int32_t ncg1 = a.d.ncg1;  // pass 1: the column groups of a row block in a row
  for (int64_t i = i0; i < a.ntiles1; i += stride)
    a.c.tiles1[i] = Tile{0, static_cast<int32_t>(i / ncg1), static_cast<int32_t>(i % ncg1), 0};
  for (int64_t i = i0; i < a.ntiles2; i += stride)
    a.c.tiles2[i] = Tile{0, static_cast<int32_t>(i % nrb), static_cast<int32_t>(i / nrb), 0};
  for (int64_t i = i0; i < a.ntiles3; i += stride)
    a.c.tiles3[i] =
        Tile{0, static_cast<int32_t>(i % a.nrb3), static_cast<int32_t>(i / a.nrb3), 0};
  for (int64_t i = i0; i < a.ntiles2r; i += stride)
    a.c.tiles2r[i] = Tile{0, 0, static_cast<int32_t>(i), 0};
  for (int64_t i = i0; i < a.npgram; i += stride)
    a.c.pgram[i] = Tile{0, static_cast<int32_t>(i), 0, 0};
  for (int64_t i = i0; i < a.nqgram; i += stride)
    a.c.qgram[i] = Tile{0, static_cast<int32_t>(i), 0, 0};
}

// The caller's warm-start Q (m x r, row stride r) into the working Q (row stride R,
// columns past r zero) and, for the matrix-core ranks, Q^T (R rows of mstride
// floats, columns past m zero).
__global__ void __launch_bounds__(256)
    k_noalloc_qin(const float* __restrict__ qc, float* __restrict__ qs, float* __restrict__ qt,
                  int m, int r, int R, int mstride) {
  const int64_t total = static_cast<int64_t>(mstride) * R;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int row = static_cast<int>(i / R);
    const int k = static_cast<int>(i % R);
    const float v = (row < m && k < r) ? qc[static_cast<int64_t>(row) * r + k] : 0.f;
    if (row < m) qs[static_cast<int64_t>(row) * R + k] = v;
    if (qt) qt[static_cast<int64_t>(k) * mstride + row] = v;
  }
}

// The working P and Q (row stride R) out to the caller's n x r and m x r arrays.
__global__ void __launch_bounds__(256)
    k_noalloc_out(const float* __restrict__ ps, float* __restrict__ pc,
                  const float* __restrict__ qs, float* __restrict__ qc, int n, int m, int r,
                  int R) {
  const int64_t np = pc ? static_cast<int64_t>(n) * r : 0;
  const int64_t total = np + static_cast<int64_t>(m) * r;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (i < np) {
      pc[i] = ps[(i / r) * R + i % r];
    } else {
      const int64_t j = i - np;
      qc[j] = qs[(j / r) * R + j % r];
    }
  }
}

unsigned grid_for(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return static_cast<unsigned>(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

}  // namespace
}  // namespace psgd

using namespace psgd;

extern "C" POWERSGD_API powersgd_status powersgd_compress_matrix_noalloc(
    const powersgd_hparams* hp, int64_t bucket_index, int32_t view, uint64_t epoch, float* M,
    int64_t n, int64_t m, float* E, float* Q, int32_t q_valid, float* P, void* stream) {
  if (!hp || !M || !Q) return report_error(POWERSGD_ERR_INVALID_ARG, "NULL hp, M or Q");
  if (n < 1 || m < 1) return report_error(POWERSGD_ERR_INVALID_ARG, "n and m must be >= 1");
  if (view < 0) return report_error(POWERSGD_ERR_INVALID_ARG, "view < 0");
  if (hp->matrix_approximation_rank < 1)
    return report_error(POWERSGD_ERR_INVALID_ARG, "matrix_approximation_rank must be >= 1");
  if (hp->matrix_approximation_rank > POWERSGD_MAX_RANK)
    return report_error(POWERSGD_ERR_UNSUPPORTED, "matrix_approximation_rank above 32");
  if (!std::isfinite(hp->orthogonalization_epsilon) || hp->orthogonalization_epsilon < 0.0)
    return report_error(POWERSGD_ERR_INVALID_ARG,
                        "orthogonalization_epsilon must be finite and >= 0");
  for (const void* p : {static_cast<const void*>(M), static_cast<const void*>(E),
                        static_cast<const void*>(Q), static_cast<const void*>(P)})
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0)
      return report_error(POWERSGD_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  MatrixLayout L;
  powersgd_status st = matrix_layout(*hp, n, m, L);
  if (st != POWERSGD_OK) return st;
  // 16-byte row accesses when the rows and both row-major arrays allow them
  const bool aligned = reinterpret_cast<uintptr_t>(M) % 16 == 0 &&
                       (E == nullptr || reinterpret_cast<uintptr_t>(E) % 16 == 0);
  if (!aligned) L.d.vec = 0;

  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return report_error(POWERSGD_ERR_HIP, hipGetErrorString(e));
  if (device < 0 || device >= kMaxDevices)
    return report_error(POWERSGD_ERR_UNSUPPORTED, "device index above 63");
  void* base = nullptr;
  e = scratch_address(device, &base);
  if (e != hipSuccess) return report_error(POWERSGD_ERR_HIP, hipGetErrorString(e));
  const Carve c = carve(static_cast<unsigned char*>(base), L);
  if (c.bytes > kScratchBytes)
    return report_error(POWERSGD_ERR_UNSUPPORTED,
                        "the matrix needs more working memory than the 64 MiB array holds");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = L.R;
  const int r = L.d.rank;
  const bool ef = E != nullptr;
  const bool fused = R <= kMaxFusedGramRank;
  const double eps = hp->orthogonalization_epsilon;
  auto check = [&](hipError_t err, const char* what) -> bool {
    if (err == hipSuccess) return true;
    report_error(POWERSGD_ERR_HIP, what);
    return false;
  };

  {
    SetupArgs a{L.d, L.pjob, L.qjob, L.qinit, L.ntiles1, L.ntiles2, L.ntiles3,
                L.ntiles2r, L.npgram, L.nqgram, L.nrb3, c};
    a.qinit.view = view;
    const int64_t most = std::max<int64_t>({L.ntiles1, L.ntiles2, L.ntiles3, 1});
    k_noalloc_setup<<<grid_for(most), 256, 0, s>>>(a);
    if (!check(hipGetLastError(), "table setup launch")) return POWERSGD_ERR_HIP;
  }
  if (q_valid) {
    k_noalloc_qin<<<grid_for(static_cast<int64_t>(L.d.mstride) * R), 256, 0, s>>>(
        Q, c.Q, c.QT, L.d.m, r, R, L.d.mstride);
    if (!check(hipGetLastError(), "warm Q copy launch")) return POWERSGD_ERR_HIP;
  } else {
    // step 3.1: the seeded N(0, 1) draw, orthogonalized
    if (!check(launch_qinit(R, c.qinit, 1, static_cast<int64_t>(L.d.m) * r, c.Q,
                            hp->random_seed, static_cast<uint64_t>(bucket_index), epoch,
                            kStF32, s), "q_init launch") ||
        !check(launch_gram(R, c.qgram, L.nqgram, c.qjob, c.Q, nullptr, c.gram, nullptr, kStF32, s),
               "Gram of Q launch") ||
        !check(launch_orth(R, c.qjob, 1, L.d.m, c.Q, c.QT, c.gram, c.tmat, eps, nullptr,
                           kStF32, s), "orthogonalize Q launch"))
      return POWERSGD_ERR_HIP;
  }
  {
    Pass1Args a{};
    a.tiles = c.tiles1;
    a.ntiles = L.ntiles1;
    a.td = c.desc;
    a.bucket = M;
    a.E = E;
    a.Q = c.Q;
    a.QT = c.QT;
    a.P = fused ? c.Praw : c.P;
    a.Ppart = c.Ppart;
    a.gram = c.gram;
    a.inv_scale = 1.0f;
    if (!check(launch_pass1(R, false, ef, kStF32, a, s), "pass 1 launch")) return POWERSGD_ERR_HIP;
  }
  if (!fused) {
    if (!check(launch_gram(R, c.pgram, L.npgram, c.pjob, c.P, c.Ppart, c.gram, nullptr, kStF32, s),
               "Gram of P launch") ||
        !check(launch_orth(R, c.pjob, 1, L.d.n, c.P, nullptr, c.gram, c.tmat, eps, nullptr,
                           kStF32, s), "orthogonalize P launch"))
      return POWERSGD_ERR_HIP;
  }
  {
    Pass2Args a{};
    a.tiles = c.tiles2;
    a.ntiles = L.ntiles2;
    a.td = c.desc;
    a.bucket = M;
    a.E = E;
    a.P = fused ? c.Praw : c.P;
    a.Pout = c.P;
    a.gram = c.gram;
    a.eps = eps;
    a.Q = c.Q;
    a.QT = c.QT;
    a.partial = c.partial;
    a.inv_scale = 1.0f;
    if (!check(launch_pass2(R, false, ef, kStF32, false, a, s), "pass 2 launch"))
      return POWERSGD_ERR_HIP;
  }
  if (!fused && L.ntiles2r > 0) {
    Pass2ReduceArgs b{};
    b.tiles = c.tiles2r;
    b.ntiles = L.ntiles2r;
    b.td = c.desc;
    b.partial = c.partial;
    b.Q = c.Q;
    b.QT = c.QT;
    if (!check(launch_pass2_reduce(R, kStF32, b, s), "pass 2 reduce launch"))
      return POWERSGD_ERR_HIP;
  }
  {
    Pass3Args a{};
    a.tiles = c.tiles3;
    a.ntiles = L.ntiles3;
    a.td = c.desc;
    a.bucket = M;
    a.E = E;
    a.P = c.P;
    a.Q = c.Q;
    a.partial = c.partial;
    a.inv_scale = 1.0f;
    if (!check(launch_pass3(R, false, ef, kStF32, a, s), "pass 3 launch")) return POWERSGD_ERR_HIP;
    if (ef) {
      // pass 1 left M' in E's place (the caller's E): the error itself goes back there
      a.Eout = E;
      if (!check(launch_error_materialize(R, kStF32, a, s), "error materialization launch"))
        return POWERSGD_ERR_HIP;
    }
  }
  k_noalloc_out<<<grid_for((P ? L.d.n : 0) * static_cast<int64_t>(r) +
                           static_cast<int64_t>(L.d.m) * r), 256, 0, s>>>(
      c.P, P, c.Q, Q, L.d.n, L.d.m, r, R);
  if (!check(hipGetLastError(), "factor copy launch")) return POWERSGD_ERR_HIP;
  return POWERSGD_OK;
}
