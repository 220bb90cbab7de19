// Host runtime of the PowerSGD bucket-compression library: the C ABI of
// include/powersgd.h, per-bucket plans (view classification, rate decisions,
// work-item tables), device memory ownership and the launch sequence.
//
// Method: "DDP Communication Hooks -- PyTorch 1.11.0", section "PowerSGD State"
// (hyperparameters, rate test, epsilon, the warning on rebuilt buckets) and section
// "PowerSGD Hooks" (powerSGD_hook steps 1 to 3.7, error-feedback memory), on one
// rank; fp16 unscale and inf skip from "torch.cuda.amp -- PyTorch 1.5.0", section
// "Gradient Scaling".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <list>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "internal.h"
#include "powersgd.h"

using namespace psgd;

namespace {

thread_local std::string g_last_error;

powersgd_status fail(powersgd_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

powersgd_status hip_fail(hipError_t e, const char* what) {
  return fail(POWERSGD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Rate test of the "PowerSGD State" section, (n + m) * rank * rate < n * m, evaluated
// exactly on the binary64 value of rate, written as mant * 2^e with an integer mant.
bool should_compress(int64_t n, int64_t m, int64_t rank, double rate) {
  if (n <= 0 || m <= 0) return false;
  using i128 = __int128;
  const i128 nm = static_cast<i128>(n) * m;              // < 2^63 (inside the bucket)
  if (rate <= 0.0) return true;                          // left side <= 0 < n * m
  int e = 0;
  const double fr = std::frexp(rate, &e);                // rate = fr * 2^e, fr in [0.5, 1)
  const int64_t mant = static_cast<int64_t>(std::ldexp(fr, 53));  // exact, < 2^53
  e -= 53;                                               // rate = mant * 2^e
  const i128 a = static_cast<i128>(n + m) * rank * mant;  // < 2^64 * 2^5 * 2^53
  if (e >= 0) {
    // a * 2^e < nm  <=>  a <= (nm - 1) >> e
    if (e >= 126) return false;
    return a <= ((nm - 1) >> e);
  }
  // a < nm * 2^-e; when the right side exceeds 2^125 it exceeds every a
  const int sh = -e;
  int bits = 0;
  for (i128 t = nm; t > 0; t >>= 1) ++bits;
  if (bits + sh >= 125) return true;
  return a < (nm << sh);
}

struct HipDeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit HipDeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~HipDeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

template <typename T>
powersgd_status upload(const std::vector<T>& v, T** dst, hipStream_t s) {
  *dst = nullptr;
  if (v.empty()) return POWERSGD_OK;
  const size_t bytes = v.size() * sizeof(T);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(dst), bytes);
  if (e != hipSuccess) return fail(POWERSGD_ERR_OOM, "hipMalloc of a work table failed");
  e = hipMemcpyAsync(*dst, v.data(), bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync of a work table");
  return POWERSGD_OK;
}

struct ViewKey {
  int64_t offset;
  std::vector<int64_t> shape;
  bool operator==(const ViewKey& o) const { return offset == o.offset && shape == o.shape; }
};

// Everything derived from one bucket layout, plus the memory the method keeps for it.
struct BucketPlan {
  int64_t numel = 0;      // bucket length (batched: the logical length, before padding)
  bool batched = false;   // the whole bucket viewed as one padded square matrix
  int st = kStF32;        // state precision (16-bit for the wrapped hook)
  std::vector<ViewKey> views;
  std::vector<uint8_t> decision;        // per view: 1 = compressed
  std::vector<int32_t> view_tensor;     // per view: tensor index or -1
  std::vector<int64_t> view_n, view_m;  // matrix shape (0 for vectors)
  std::vector<int32_t> view_rank;
  int R = 1;
  int64_t compressed_elems = 0;
  int64_t uncompressed_elems = 0;
  int64_t comm_elems = 0;
  int64_t all_elems = 0;
  std::vector<TensorDesc> tensors;
  std::vector<Tile> tiles1, tiles2, tiles3, tiles2r;
  std::vector<FlatTile> flat_unc, flat_all;
  std::vector<OrthJob> pjobs, qjobs;
  std::vector<Tile> pgram_tiles, qgram_tiles;  // (job, partial) for the Gram kernel
  std::vector<QInitJob> qinit;
  int64_t max_qcount = 0;
  int max_prows = 0, max_qrows = 0;
  int64_t e_floats = 0, p_floats = 0, q_floats = 0, partial_floats = 0, gram_doubles = 0;
  int64_t ppart_floats = 0;  // matrix-core ranks: pass 1's column-group partials of P
  int64_t qt_floats = 0;

  // device memory
  float* E = nullptr;
  uint16_t* Eh = nullptr;  // 16-bit state with error feedback: E's place (M' or the error)
  uint16_t* Mh = nullptr;  // 16-bit state without error feedback: M' of the current call
  float* P = nullptr;
  float* Praw = nullptr;  // vector ranks: P as pass 1 writes it (pass 2 orthogonalizes)
  float* Ppart = nullptr;  // matrix-core ranks: pass 1's column-group partials of P
  float* Q = nullptr;
  float* QT = nullptr;  // matrix-core ranks: Q transposed
  float* partial = nullptr;
  double* gram = nullptr;
  double* tmat = nullptr;  // the r x r transform of each orthogonalization job
  Tile* d_pgram_tiles = nullptr;
  Tile* d_qgram_tiles = nullptr;
  TensorDesc* d_td = nullptr;         // rows vector-aligned where possible
  TensorDesc* d_td_scalar = nullptr;  // same with every vec flag cleared
  Tile* d_tiles1 = nullptr;   // pass 1 row blocks
  Tile* d_tiles2 = nullptr;   // pass 2 (row block, column block)
  Tile* d_tiles3 = nullptr;   // pass 3 (row block, column block)
  Tile* d_tiles2r = nullptr;  // pass-2 partial sums (column blocks of split tensors)
  FlatTile* d_flat_unc = nullptr;
  FlatTile* d_flat_all = nullptr;
  OrthJob* d_pjobs = nullptr;
  OrthJob* d_qjobs = nullptr;
  QInitJob* d_qinit = nullptr;
  // introspection copies (allocated on first use): the bucket-shaped E of
  // powersgd_get_error and the compact factors of powersgd_get_factors
  float* intro_E = nullptr;
  float* intro_PQ = nullptr;
  std::vector<int64_t> intro_off;  // per tensor: first float of its compact P, then Q
  hipStream_t last_stream = nullptr;  // stream of the latest compressing call
  // E's place (the error memory, fp32 or 16-bit) is known to hold the error itself
  // (true: before the first call, after an import, after a materialization in place);
  // false after a call that keeps M' there (an fp16 step skipped for inf leaves the
  // error in place: the device flag wflag says which, for the kernels)
  bool w_holds_e = true;
  int32_t* wflag = nullptr;  // device: non-zero while E's place holds the error itself
  // fp32 state created by an fp16 call: E's place is two buffers wstride floats apart,
  // the device index widx naming the current one; a step's pass 1 writes M' into the
  // other and pass 3 of a step that ran switches them, so a step skipped for inf leaves
  // M'_prev untouched without checking the bucket first (wstride 0: one buffer)
  int32_t* widx = nullptr;
  int64_t wstride = 0;
  float* Emat = nullptr;  // the materialized error for introspection and export
  bool allocated = false;
  bool q_ready = false;
  // every tensor has 16-byte aligned rows (in d_td) at least 256 columns wide
  bool all_wide = false;

  // A 16-bit state's M' of the call, as the passes read and write it: E's place with
  // error feedback (pass 1 replaces M'_prev there), the separate array without.
  uint16_t* mprime16() const { return Eh ? Eh : Mh; }
  // E's place holds M' of the previous call (a state with error feedback)
  bool keeps_mprime() const { return E != nullptr || Eh != nullptr; }

  void release() {
    void* ptrs[] = {E, Eh, Mh, P, Praw, Ppart, Q, QT, partial, gram, tmat, d_pgram_tiles, d_qgram_tiles, d_td, d_td_scalar,
                    d_tiles1, d_tiles2, d_tiles3, d_tiles2r, d_flat_unc, d_flat_all, d_pjobs, d_qjobs,
                    d_qinit, intro_E, intro_PQ, Emat, wflag, widx};
    for (void* p : ptrs)
      if (p) (void)hipFree(p);
    E = P = Praw = Ppart = Q = QT = partial = nullptr;
    Eh = Mh = nullptr;
    gram = nullptr;
    tmat = nullptr;
    d_pgram_tiles = d_qgram_tiles = nullptr;
    d_td = d_td_scalar = nullptr;
    d_tiles1 = d_tiles2 = d_tiles3 = d_tiles2r = nullptr;
    d_flat_unc = d_flat_all = nullptr;
    d_pjobs = d_qjobs = nullptr;
    d_qinit = nullptr;
    intro_E = intro_PQ = Emat = nullptr;
    wflag = nullptr;
    widx = nullptr;
    wstride = 0;
    intro_off.clear();
    allocated = false;
  }
  ~BucketPlan() { release(); }
};

constexpr int64_t kFlatChunk = 1 << 16;

void add_flat(std::vector<FlatTile>& out, int64_t start, int64_t len) {
  for (int64_t s = 0; s < len; s += kFlatChunk)
    out.push_back(FlatTile{start + s, std::min(kFlatChunk, len - s)});
}

struct TimingRec {
  int kind;
  hipEvent_t start, stop;
  double bytes;
};

}  // namespace

struct powersgd_state {
  powersgd_hparams hp;
  int device = 0;
  int64_t iteration = 0;
  int64_t numel_in = 0;
  int64_t numel_comm = 0;
  int64_t next_log_iteration = 0;
  std::map<int64_t, std::unique_ptr<BucketPlan>> buckets;
  std::map<int64_t, std::unique_ptr<BucketPlan>> passthrough;  // fp16 unscale tables only
  hipStream_t last_stream = nullptr;
  // timing
  bool timing = false;
  std::vector<TimingRec> pending;
  std::vector<hipEvent_t> free_events;
  double t_ms[POWERSGD_NUM_KERNELS] = {};
  int64_t t_count[POWERSGD_NUM_KERNELS] = {};
  double t_bytes[POWERSGD_NUM_KERNELS] = {};
};

namespace {

enum KernelKind {
  K_QINIT = 0, K_PASS1 = 1, K_ORTH = 2, K_PASS2 = 3, K_PASS3 = 4, K_UNSCALE = 5, K_PASS2R = 6,
  K_GRAM = 7
};

hipEvent_t take_event(powersgd_state* st) {
  if (!st->free_events.empty()) {
    hipEvent_t e = st->free_events.back();
    st->free_events.pop_back();
    return e;
  }
  // timing only: no system-scope fence (cache writeback) when the event is recorded,
  // so the events disturb the kernels they bracket as little as possible
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Drains recorded events into the per-kernel totals (waits for them).
void collect_timing(powersgd_state* st) {
  for (TimingRec& r : st->pending) {
    (void)hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      st->t_ms[r.kind] += ms;
      st->t_count[r.kind] += 1;
      st->t_bytes[r.kind] += r.bytes;
    }
    st->free_events.push_back(r.start);
    st->free_events.push_back(r.stop);
  }
  st->pending.clear();
}

// Runs one launch, bracketed by events when timing is on.
template <typename F>
powersgd_status timed_launch(powersgd_state* st, hipStream_t s, int kind, double bytes,
                             const char* what, F&& launch) {
  TimingRec rec{kind, nullptr, nullptr, bytes};
  if (st->timing) {
    if (st->pending.size() > 4096) collect_timing(st);
    rec.start = take_event(st);
    rec.stop = take_event(st);
    if (rec.start && rec.stop) (void)hipEventRecord(rec.start, s);
  }
  const hipError_t e = launch();
  if (e != hipSuccess) return hip_fail(e, what);
  if (st->timing && rec.start && rec.stop) {
    (void)hipEventRecord(rec.stop, s);
    st->pending.push_back(rec);
  }
  return POWERSGD_OK;
}

powersgd_status validate_views(const powersgd_view* views, int32_t nviews, int64_t numel,
                               std::vector<ViewKey>& out) {
  out.clear();
  out.reserve(nviews);
  std::vector<std::pair<int64_t, int64_t>> ranges;
  for (int32_t v = 0; v < nviews; ++v) {
    const powersgd_view& pv = views[v];
    if (pv.ndim < 0 || pv.ndim > POWERSGD_MAX_NDIM)
      return fail(POWERSGD_ERR_INVALID_ARG, "view " + std::to_string(v) + ": ndim out of range");
    ViewKey k;
    k.offset = pv.offset;
    int64_t size = 1;
    for (int64_t d = 0; d < pv.ndim; ++d) {
      const int64_t s = pv.shape[d];
      if (s < 0) return fail(POWERSGD_ERR_INVALID_ARG, "view " + std::to_string(v) + ": negative dimension");
      if (s > 0 && size > INT64_MAX / s)
        return fail(POWERSGD_ERR_INVALID_ARG, "view " + std::to_string(v) + ": size overflows");
      size *= s;
      k.shape.push_back(s);
    }
    if (pv.offset < 0 || pv.offset > numel || size > numel - pv.offset)
      return fail(POWERSGD_ERR_INVALID_ARG, "view " + std::to_string(v) + ": outside the bucket");
    if (size > 0) ranges.emplace_back(pv.offset, pv.offset + size);
    out.push_back(std::move(k));
  }
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second)
      return fail(POWERSGD_ERR_INVALID_ARG, "views overlap");
  return POWERSGD_OK;
}

int64_t view_numel(const ViewKey& k) {
  int64_t s = 1;
  for (int64_t d : k.shape) s *= d;
  return s;
}

// Classification, rate decisions and work tables for one layout (host only).
powersgd_status build_plan(const powersgd_hparams& hp, int64_t numel, bool batched, int prec,
                           std::vector<ViewKey>&& views, BucketPlan& pl) {
  pl.numel = numel;
  pl.batched = batched;
  pl.st = prec;
  pl.views = std::move(views);
  const size_t nv = pl.views.size();
  pl.decision.assign(nv, 0);
  pl.view_tensor.assign(nv, -1);
  pl.view_n.assign(nv, 0);
  pl.view_m.assign(nv, 0);
  pl.view_rank.assign(nv, 0);
  int max_rank = 1;
  for (size_t v = 0; v < nv; ++v) {
    const ViewKey& k = pl.views[v];
    const int64_t size = view_numel(k);
    pl.all_elems += size;
    bool comp = false;
    if (k.shape.size() >= 2) {
      const int64_t n = k.shape[0];
      const int64_t m = n > 0 ? size / n : 0;
      const int64_t rank = std::min<int64_t>(hp.matrix_approximation_rank, std::min(n, m));
      // the batched variant compresses its one square matrix without a rate test
      comp = batched ? (n > 0 && m > 0) : should_compress(n, m, rank, hp.min_compression_rate);
      if (comp) {
        if (n > kMaxMatrixDim || m > kMaxMatrixDim)
          return fail(POWERSGD_ERR_UNSUPPORTED, "matrix dimension above 2^31 - 65537");
        pl.view_n[v] = n;
        pl.view_m[v] = m;
        pl.view_rank[v] = static_cast<int32_t>(rank);
        max_rank = std::max<int>(max_rank, static_cast<int>(rank));
      }
    }
    pl.decision[v] = comp ? 1 : 0;
    if (comp) {
      pl.compressed_elems += size;
      pl.comm_elems += (pl.view_n[v] + pl.view_m[v]) * pl.view_rank[v];
    } else {
      pl.uncompressed_elems += size;
      pl.comm_elems += size;
      add_flat(pl.flat_unc, k.offset, size);
    }
    add_flat(pl.flat_all, k.offset, size);
  }
  if (batched) pl.all_elems = numel;  // statistics count the bucket, not its padding
  pl.R = pow2_ceil(max_rank);
  const int R = pl.R;

  // Work-item size: enough workgroups to fill 256 CUs several times over, and no
  // more than 64K elements (256 KB of fp32) each.
  const int64_t target =
      std::min<int64_t>(1 << 16, std::max<int64_t>(1 << 13, pl.compressed_elems / PSGD_TILES_PER_BUCKET));
  const int64_t unroll1 = pass1_unroll(R);
  // pass 1 of a 16-bit state moves 8 B per element: twice as many work items
  const int64_t target1 = prec != kStF32 ? std::max<int64_t>(1 << 13, target / 2) : target;
  const int64_t ng = static_cast<int64_t>(R) * (R + 1) / 2;
  const bool fused_gram = R <= kMaxFusedGramRank;
  // a 16-bit state's pass-2 work item carries half the bytes of an fp32 one for the same
  // orthogonalization prologue: twice the rows, where the bucket is large enough to be
  // sized above the element floor (a smaller one would run too few work items)
  const int64_t h16_scale = (prec != kStF32 && target > (1 << 13)) ? 2 : 1;
  int64_t goff = 0;
  int64_t eoff = 0, poff = 0, qoff = 0, qtoff = 0, p1off = 0;
  int32_t pslot = 0;
  for (size_t v = 0; v < nv; ++v) {
    if (!pl.decision[v]) continue;
    TensorDesc d{};
    d.boff = pl.views[v].offset;
    d.n = static_cast<int32_t>(pl.view_n[v]);
    d.m = static_cast<int32_t>(pl.view_m[v]);
    d.rank = pl.view_rank[v];
    d.vec = (d.boff % 4 == 0 && d.m % 4 == 0) ? 1 : 0;
    d.view = static_cast<int32_t>(v);
    d.eoff = eoff;
    d.poff = poff;
    d.qoff = qoff;
    eoff += round_up(static_cast<int64_t>(d.n) * d.m, 64);
    poff += round_up(static_cast<int64_t>(d.n) * R, 64);
    qoff += round_up(static_cast<int64_t>(d.m) * R, 64);
    d.mstride = static_cast<int32_t>(round_up(d.m, 4));
    d.qtoff = -1;
    if (R >= kMfmaMinRank) {
      d.qtoff = qtoff;
      qtoff += round_up(static_cast<int64_t>(d.mstride) * R, 64);
    }
    const int32_t ti = static_cast<int32_t>(pl.tensors.size());
    // pass 1: whole rows; slots of lprw threads sweep 4 * lprw columns at a time
    // (matrix-core ranks: 32-row blocks split into groups of kPass1Cols columns, the
    // groups of a row block next to each other in the table, each writing a partial P)
    d.lprw = pow2_ceil(static_cast<int>((std::min<int64_t>(d.m, 4 * kThreads) + 3) / 4));
    {
      int64_t rows;
      if (R >= kMfmaMinRank) {
        rows = kMfmaPass1Rows;
      } else {
        const int64_t slots = kThreads / d.lprw;
        rows = round_up(std::max<int64_t>(1, (target1 + d.m - 1) / d.m), slots * unroll1);
        rows = std::min<int64_t>(rows, round_up(d.n, slots));
        if (d.lprw > 64) {
          // the wavefront sums of every row of the tile are parked in LDS
          const int64_t wps = d.lprw / 64;
          const int64_t step = slots * unroll1;
          rows = std::min<int64_t>(rows, kPass1SlotSums / wps / step * step);
        }
      }
      d.rpb1 = static_cast<int32_t>(rows);
      d.ncg1 = 1;
      d.p1off = 0;
      if (R >= kMfmaMinRank) {
        d.ncg1 = static_cast<int32_t>((d.m + kPass1Cols - 1) / kPass1Cols);
        d.p1off = p1off;
        p1off += round_up(static_cast<int64_t>(d.ncg1) * d.n * R, 64);
      }
      for (int64_t r0 = 0, rb = 0; r0 < d.n; r0 += rows, ++rb)
        for (int32_t cg = 0; cg < d.ncg1; ++cg)
          pl.tiles1.push_back(Tile{ti, static_cast<int32_t>(rb), cg, 0});
    }
    // Gram partials of P: one per pass-1 row block (fused) or per kGramRows rows
    {
      const int32_t rpp = fused_gram ? d.rpb1 : kGramRows;
      const int32_t nparts = static_cast<int32_t>((d.n + rpp - 1) / rpp);
      d.goff = goff;
      // matrix-core ranks: the Gram kernel first sums pass 1's column-group partials
      pl.pjobs.push_back(OrthJob{d.poff, goff, -1, d.n, d.rank, nparts, rpp, 0,
                                 R >= kMfmaMinRank ? d.ncg1 : 0, d.p1off});
      if (!fused_gram)
        for (int32_t pp = 0; pp < nparts; ++pp)
          pl.pgram_tiles.push_back(Tile{static_cast<int32_t>(pl.pjobs.size() - 1), pp, 0, 0});
      // pass 1's partials are fp64; the Gram kernel's are double-double
      goff += nparts * ng * (fused_gram ? 1 : 2);
    }
    // pass 2 / pass 3: (row block) x (256-column block)
    const int64_t width = std::min<int64_t>(d.m, kColBlock);
    d.lpr = pow2_ceil(static_cast<int>((width + 3) / 4));
    const int64_t rpw = 64 / d.lpr;
    auto row_block = [&](int64_t tgt) {
      int64_t rb = round_up(std::max<int64_t>(1, (tgt + width - 1) / width), 16 * rpw);
      rb = std::min<int64_t>(rb, round_up(d.n, 4 * rpw));
      if (R >= kMfmaMinRank) rb = std::min<int64_t>(kMfmaRowBlock, round_up(d.n, 16));
      return rb;
    };
    // vector ranks: every pass-2 workgroup orthogonalizes its P rows first, so its
    // work items are larger (fewer of them pay that prologue) and its rows fit in LDS
    int64_t rpb = row_block(fused_gram ? std::min<int64_t>(h16_scale << 16,
                                                           target * PSGD_PASS2_TILE_SCALE * h16_scale)
                                       : target);
    if (R >= kMfmaMinRank) rpb = std::min<int64_t>(kMfmaPass2Rows, round_up(d.n, 16));
    if (fused_gram) rpb = std::min<int64_t>(rpb, kPass2StageFloats / R);
    d.rpb = static_cast<int32_t>(rpb);
    d.nrb = static_cast<int32_t>((d.n + rpb - 1) / rpb);
    // vector ranks: every pass-3 work item first sums the pass-2 partial slots of its
    // column block, so taller items pay that less often
    d.rpb3 = static_cast<int32_t>(
        row_block(R <= kMaxFusedGramRank ? target * PSGD_PASS3_TILE_SCALE : target));
    const int32_t nrb3 = (d.n + d.rpb3 - 1) / d.rpb3;
    d.ncb = static_cast<int32_t>((d.m + kColBlock - 1) / kColBlock);
    if (d.nrb > 1) {
      d.pslot = pslot;
      pslot += d.nrb * d.ncb;
      for (int32_t cb = 0; cb < d.ncb; ++cb) pl.tiles2r.push_back(Tile{ti, 0, cb, 0});
    }
    pl.view_tensor[v] = ti;
    for (int32_t cb = 0; cb < d.ncb; ++cb) {
      for (int32_t rb = 0; rb < d.nrb; ++rb) pl.tiles2.push_back(Tile{ti, rb, cb, 0});
      for (int32_t rb = 0; rb < nrb3; ++rb) pl.tiles3.push_back(Tile{ti, rb, cb, 0});
    }
    {
      const int32_t nparts = static_cast<int32_t>((d.m + kGramRows - 1) / kGramRows);
      pl.qjobs.push_back(
          OrthJob{d.qoff, goff, d.qtoff, d.m, d.rank, nparts, kGramRows, d.mstride, 0, 0});
      for (int32_t pp = 0; pp < nparts; ++pp)
        pl.qgram_tiles.push_back(Tile{static_cast<int32_t>(pl.qjobs.size() - 1), pp, 0, 0});
      goff += nparts * ng * 2;  // double-double partials
    }
    pl.qinit.push_back(QInitJob{d.qoff, d.m, d.rank, d.view, 0});
    pl.max_qcount = std::max<int64_t>(pl.max_qcount, static_cast<int64_t>(d.m) * d.rank);
    pl.max_prows = std::max(pl.max_prows, d.n);
    pl.max_qrows = std::max(pl.max_qrows, d.m);
    pl.tensors.push_back(d);
  }
  pl.all_wide = !pl.tensors.empty();
  for (const TensorDesc& d : pl.tensors) pl.all_wide = pl.all_wide && d.vec && d.lpr == 64;
  pl.e_floats = eoff;
  pl.p_floats = poff;
  pl.q_floats = qoff;
  pl.partial_floats = static_cast<int64_t>(pslot) * kColBlock * R;
  pl.ppart_floats = p1off;
  pl.gram_doubles = goff;
  pl.qt_floats = qtoff;
  if (R <= kMaxFusedGramRank) {
    // Vector ranks: every pass-3 work item sums the pass-2 partial slots of its column
    // block. The dispatcher deals workgroups to the 8 XCDs in turn (workgroup b to XCD
    // b % 8), each with its own L2; workgroup b takes the item at position start(b % 8)
    // + b / 8 of the list, so that each XCD works through one contiguous eighth of it
    // and the items of a column block share one L2 (the matrix-core pass 3 was measured
    // slower in this order).
    const size_t n = pl.tiles3.size(), X = 8;
    std::vector<Tile> out(n);
    size_t start = 0;
    for (size_t x = 0; x < X; ++x) {
      const size_t cnt = n / X + (x < n % X ? 1 : 0);
      for (size_t k = 0; k < cnt; ++k) out[x + X * k] = pl.tiles3[start + k];
      start += cnt;
    }
    pl.tiles3.swap(out);
  }
  return POWERSGD_OK;
}

powersgd_status allocate_plan(BucketPlan& pl, bool need_e, bool double_w, hipStream_t s) {
  auto alloc = [&](void** p, size_t bytes) -> bool {
    if (bytes == 0) {
      *p = nullptr;
      return true;
    }
    return hipMalloc(p, bytes) == hipSuccess;
  };
  bool ok = true;
  const bool h16 = pl.st != kStF32;
  double_w = double_w && need_e && !h16 && pl.e_floats > 0;
  ok = ok && alloc(reinterpret_cast<void**>(&pl.E),
                   (need_e && !h16) ? (double_w ? 2 : 1) * pl.e_floats * sizeof(float) : 0);
  ok = ok && alloc(reinterpret_cast<void**>(&pl.Eh),
                   (need_e && h16) ? pl.e_floats * sizeof(uint16_t) : 0);
  ok = ok && alloc(reinterpret_cast<void**>(&pl.Mh),
                   (h16 && !need_e) ? pl.e_floats * sizeof(uint16_t) : 0);
  ok = ok && alloc(reinterpret_cast<void**>(&pl.P), pl.p_floats * sizeof(float));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.Praw),
                   pl.R <= kMaxFusedGramRank ? pl.p_floats * sizeof(float) : 0);
  ok = ok && alloc(reinterpret_cast<void**>(&pl.Q), pl.q_floats * sizeof(float));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.QT), pl.qt_floats * sizeof(float));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.partial), pl.partial_floats * sizeof(float));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.Ppart), pl.ppart_floats * sizeof(float));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.gram), pl.gram_doubles * sizeof(double));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.tmat),
                   pl.tensors.size() * static_cast<size_t>(pl.R) * pl.R * sizeof(double));
  ok = ok && alloc(reinterpret_cast<void**>(&pl.wflag), (pl.E || pl.Eh) ? sizeof(int32_t) : 0);
  ok = ok && alloc(reinterpret_cast<void**>(&pl.widx), double_w ? sizeof(int32_t) : 0);
  pl.wstride = double_w ? pl.e_floats : 0;

  if (!ok) {
    pl.release();
    return fail(POWERSGD_ERR_OOM, "device allocation of the bucket state failed");
  }
  hipError_t e = hipSuccess;
  if (pl.E && e == hipSuccess)
    e = hipMemsetAsync(pl.E, 0, (pl.wstride ? 2 : 1) * pl.e_floats * sizeof(float), s);
  if (pl.Eh && e == hipSuccess) e = hipMemsetAsync(pl.Eh, 0, pl.e_floats * sizeof(uint16_t), s);
  if (pl.Mh && e == hipSuccess) e = hipMemsetAsync(pl.Mh, 0, pl.e_floats * sizeof(uint16_t), s);
  if (pl.P && e == hipSuccess) e = hipMemsetAsync(pl.P, 0, pl.p_floats * sizeof(float), s);
  if (pl.Praw && e == hipSuccess)
    e = hipMemsetAsync(pl.Praw, 0, pl.p_floats * sizeof(float), s);
  if (pl.Q && e == hipSuccess) e = hipMemsetAsync(pl.Q, 0, pl.q_floats * sizeof(float), s);
  if (pl.QT && e == hipSuccess) e = hipMemsetAsync(pl.QT, 0, pl.qt_floats * sizeof(float), s);
  if (pl.wflag && e == hipSuccess) e = launch_set_flag(pl.wflag, 1, s);  // E = 0 in place
  if (pl.widx && e == hipSuccess) e = launch_set_flag(pl.widx, 0, s);

  if (e != hipSuccess) {
    pl.release();
    return hip_fail(e, "hipMemsetAsync of the bucket state");
  }
  std::vector<TensorDesc> scalar = pl.tensors;
  for (TensorDesc& d : scalar) d.vec = 0;
  powersgd_status st = POWERSGD_OK;
  if (st == POWERSGD_OK) st = upload(pl.tensors, &pl.d_td, s);
  if (st == POWERSGD_OK) st = upload(scalar, &pl.d_td_scalar, s);
  if (st == POWERSGD_OK) st = upload(pl.tiles1, &pl.d_tiles1, s);
  if (st == POWERSGD_OK) st = upload(pl.tiles2, &pl.d_tiles2, s);
  if (st == POWERSGD_OK) st = upload(pl.tiles3, &pl.d_tiles3, s);
  if (st == POWERSGD_OK) st = upload(pl.tiles2r, &pl.d_tiles2r, s);
  if (st == POWERSGD_OK) st = upload(pl.flat_unc, &pl.d_flat_unc, s);
  if (st == POWERSGD_OK) st = upload(pl.flat_all, &pl.d_flat_all, s);
  if (st == POWERSGD_OK) st = upload(pl.pjobs, &pl.d_pjobs, s);
  if (st == POWERSGD_OK) st = upload(pl.qjobs, &pl.d_qjobs, s);
  if (st == POWERSGD_OK) st = upload(pl.qinit, &pl.d_qinit, s);
  if (st == POWERSGD_OK) st = upload(pl.pgram_tiles, &pl.d_pgram_tiles, s);
  if (st == POWERSGD_OK) st = upload(pl.qgram_tiles, &pl.d_qgram_tiles, s);
  if (st != POWERSGD_OK) {
    pl.release();
    return st;
  }
  // The host vectors above must outlive the asynchronous uploads.
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    pl.release();
    return hip_fail(e, "hipStreamSynchronize after the state upload");
  }
  pl.allocated = true;
  return POWERSGD_OK;
}

bool same_layout(const BucketPlan& pl, int64_t numel, bool batched, int prec,
                 const std::vector<ViewKey>& views) {
  return pl.numel == numel && pl.batched == batched && pl.st == prec && pl.views == views;
}

// Side of the square matrix the batched variant views a bucket of `numel` elements as:
// the smallest s with s * s >= numel.
int64_t batched_side(int64_t numel) {
  if (numel <= 0) return 0;
  using u128 = unsigned __int128;
  const u128 n = static_cast<u128>(numel);
  int64_t s = static_cast<int64_t>(std::sqrt(static_cast<double>(numel)));
  while (s > 0 && static_cast<u128>(s) * static_cast<u128>(s) >= n) --s;
  while (static_cast<u128>(s) * static_cast<u128>(s) < n) ++s;
  return s;
}

// Minimum bytes per compressed element that each pass moves. Without error feedback
// pass 3 only writes M_hat (M' is not read).
double pass_bytes(int kind, bool f16, bool ef, int prec = kStF32) {
  if (prec != kStF32) {
    // fp32 bucket, 16-bit M' (in E's place with error feedback): pass 1 reads G (and
    // M'_prev) and writes M', pass 2 reads M', pass 3 writes M_hat
    switch (kind) {
      case K_PASS1: return 4.0 + (ef ? 2.0 : 0.0) + 2.0;
      case K_PASS2: return 2.0;
      case K_PASS3: return 4.0;
      default: return 0.0;
    }
  }
  const double g = f16 ? 2.0 : 4.0;
  // fp32 state with error feedback: pass 1 reads G and M'_prev and writes M' (g + 8),
  // pass 2 reads M' (4), pass 3 writes M_hat (g); fp16 buckets add the inf check (2,
  // counted with the fp16 check kernel)
  switch (kind) {
    case K_PASS1: return ef ? g + 8.0 : g;
    case K_PASS2: return ef ? 4.0 : g;
    case K_PASS3: return g;
    default: return 0.0;
  }
}

}  // namespace

namespace {

// The error of every tensor of a plan keeping M' in E's place, on stream s: E = M'_prev -
// P Q^T with pass 3's rounding, or E's place as it is while the device flag says it holds
// the error. Written as binary32 to dst (E's layout), or, with dst NULL, back into E's
// current place (in 16 bits for a 16-bit plan).
powersgd_status materialize_error(BucketPlan& pl, float* dst, hipStream_t s) {
  Pass3Args a{};
  a.tiles = pl.d_tiles3;
  a.ntiles = static_cast<int32_t>(pl.tiles3.size());
  a.td = pl.d_td;
  a.E = pl.E;
  a.Eh = pl.Eh;
  a.Mh = pl.Eh;  // a 16-bit plan's M'_prev
  a.P = pl.P;
  a.Q = pl.Q;
  a.inv_scale = 1.0f;
  a.Eout = dst;
  a.wflag = pl.wflag;  // E's place may still hold the error itself (a skipped fp16 step)
  a.widx = pl.widx;
  a.wstride = pl.wstride;
  const hipError_t e = launch_error_materialize(pl.R, pl.st, a, s);
  if (e != hipSuccess) return hip_fail(e, "error materialization");
  return POWERSGD_OK;
}

// Device memory holding the error of a plan as binary32, E's layout: an fp32 plan's
// single E's place itself while it holds the error, else a copy materialized on stream s
// (which of two places is current is known on the device only; a 16-bit plan whose E's
// place holds the error is widened by the callers instead).
powersgd_status error_source(BucketPlan& pl, hipStream_t s, const float** out) {
  if (pl.w_holds_e && pl.E && pl.wstride == 0) {
    *out = pl.E;
    return POWERSGD_OK;
  }
  if (!pl.Emat) {
    void* p = nullptr;
    if (hipMalloc(&p, std::max<int64_t>(pl.e_floats, 1) * sizeof(float)) != hipSuccess)
      return fail(POWERSGD_ERR_OOM, "allocation of the materialized error failed");
    pl.Emat = static_cast<float*>(p);
  }
  powersgd_status r = materialize_error(pl, pl.Emat, s);
  if (r != POWERSGD_OK) return r;
  *out = pl.Emat;
  return POWERSGD_OK;
}

}  // namespace

namespace psgd {

powersgd_status report_error(powersgd_status s, const char* msg) { return fail(s, msg); }

powersgd_status matrix_layout(const powersgd_hparams& hp, int64_t n, int64_t m,
                              MatrixLayout& out) {
  if (n <= 0 || m <= 0) return fail(POWERSGD_ERR_INVALID_ARG, "the matrix is empty");
  if (n > kMaxMatrixDim || m > kMaxMatrixDim)
    return fail(POWERSGD_ERR_UNSUPPORTED, "matrix dimension above 2^31 - 65537");
  BucketPlan pl;
  std::vector<ViewKey> keys{ViewKey{0, {n, m}}};
  // the batched variant's plan: one matrix, no rate test
  powersgd_status b = build_plan(hp, n * m, true, kStF32, std::move(keys), pl);
  if (b != POWERSGD_OK) return b;
  out.d = pl.tensors[0];
  out.R = pl.R;
  out.pjob = pl.pjobs[0];
  out.qjob = pl.qjobs[0];
  out.qinit = pl.qinit[0];
  out.ntiles1 = static_cast<int32_t>(pl.tiles1.size());
  out.ntiles2 = static_cast<int32_t>(pl.tiles2.size());
  out.ntiles3 = static_cast<int32_t>(pl.tiles3.size());
  out.ntiles2r = static_cast<int32_t>(pl.tiles2r.size());
  out.npgram = static_cast<int32_t>(pl.pgram_tiles.size());
  out.nqgram = static_cast<int32_t>(pl.qgram_tiles.size());
  out.nrb3 = out.d.ncb > 0 ? out.ntiles3 / out.d.ncb : 0;
  out.p_floats = pl.p_floats;
  out.q_floats = pl.q_floats;
  out.qt_floats = pl.qt_floats;
  out.partial_floats = pl.partial_floats;
  out.ppart_floats = pl.ppart_floats;
  out.gram_doubles = pl.gram_doubles;
  return POWERSGD_OK;
}

}  // namespace psgd

// ============================================================================ ABI

extern "C" {

void powersgd_hparams_init(powersgd_hparams* hp) {
  if (!hp) return;
  std::memset(hp, 0, sizeof(*hp));
  hp->matrix_approximation_rank = 1;
  hp->start_powerSGD_iter = 1000;
  hp->min_compression_rate = 2.0;
  hp->use_error_feedback = 1;
  hp->warm_start = 1;
  hp->orthogonalization_epsilon = 0.0;
  hp->random_seed = 0;
  hp->compression_stats_logging_frequency = 10000;
  hp->batch_tensors_with_same_shape = 0;
}

const char* powersgd_status_string(powersgd_status s) {
  switch (s) {
    case POWERSGD_OK: return "ok";
    case POWERSGD_ERR_INVALID_ARG: return "invalid argument";
    case POWERSGD_ERR_LAYOUT_CHANGED: return "bucket layout changed after its state was memorized";
    case POWERSGD_ERR_OOM: return "out of device memory";
    case POWERSGD_ERR_HIP: return "HIP runtime error";
    case POWERSGD_ERR_UNSUPPORTED: return "unsupported configuration";
    case POWERSGD_ERR_NOT_FOUND: return "no such bucket or view";
  }
  return "unknown status";
}

const char* powersgd_last_error(void) { return g_last_error.c_str(); }

const char* powersgd_kernel_name(int32_t kind) {
  static const char* names[POWERSGD_NUM_KERNELS] = {
      "q_init", "pass1_mq", "orthogonalize", "pass2_mtp", "pass3_decompress_error",
      "unscale_only", "pass2_reduce", "gram"};
  if (kind < 0 || kind >= POWERSGD_NUM_KERNELS) return "";
  return names[kind];
}

powersgd_status powersgd_state_create(const powersgd_hparams* hp, int32_t device,
                                      powersgd_state** out) {
  if (!out) return fail(POWERSGD_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!hp) return fail(POWERSGD_ERR_INVALID_ARG, "hp is NULL");
  if (hp->matrix_approximation_rank < 1)
    return fail(POWERSGD_ERR_INVALID_ARG, "matrix_approximation_rank must be >= 1");
  if (hp->matrix_approximation_rank > POWERSGD_MAX_RANK)
    return fail(POWERSGD_ERR_UNSUPPORTED, "matrix_approximation_rank above 32");
  if (!std::isfinite(hp->orthogonalization_epsilon) || hp->orthogonalization_epsilon < 0.0)
    return fail(POWERSGD_ERR_INVALID_ARG, "orthogonalization_epsilon must be finite and >= 0");
  if (!std::isfinite(hp->min_compression_rate))
    return fail(POWERSGD_ERR_INVALID_ARG, "min_compression_rate must be finite");
  if (hp->start_powerSGD_iter < 0)
    return fail(POWERSGD_ERR_INVALID_ARG, "start_powerSGD_iter must be >= 0");
  if (device < 0) return fail(POWERSGD_ERR_INVALID_ARG, "device must be >= 0");
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device >= count) return fail(POWERSGD_ERR_INVALID_ARG, "no such device");
  auto* st = new (std::nothrow) powersgd_state();
  if (!st) return fail(POWERSGD_ERR_OOM, "host allocation failed");
  st->hp = *hp;
  st->device = device;
  st->next_log_iteration = hp->start_powerSGD_iter;
  *out = st;
  return POWERSGD_OK;
}

void powersgd_state_destroy(powersgd_state* st) {
  if (!st) return;
  HipDeviceGuard guard(st->device);
  (void)hipDeviceSynchronize();
  collect_timing(st);
  for (hipEvent_t e : st->free_events) (void)hipEventDestroy(e);
  st->buckets.clear();
  st->passthrough.clear();
  delete st;
}

namespace {

// One hook call on a validated bucket layout: the per-layer variant (`keys` = the
// views) or the batched one (`keys` = the one padded square view, `numel` = the
// bucket's own length).
powersgd_status run_call(powersgd_state* st, int64_t bucket_index, int32_t is_last,
                         void* bucket, bool f16, int64_t numel, bool batched, int prec,
                         std::vector<ViewKey>& keys, float inv_loss_scale,
                         int32_t* found_inf_dev, void* stream) {
  HipDeviceGuard guard(st->device);
  if (!guard.ok) return fail(POWERSGD_ERR_HIP, "hipSetDevice failed");
  hipStream_t s = static_cast<hipStream_t>(stream);
  st->last_stream = s;
  const powersgd_hparams& hp = st->hp;
  const bool ef = hp.use_error_feedback != 0;
  const uintptr_t base = reinterpret_cast<uintptr_t>(bucket);

  // Vanilla allreduce phase (iteration < start_powerSGD_iter): identity on one rank;
  // fp16 still does the unscale with its inf check, the wrapped hook the 16-bit cast.
  if (st->iteration < hp.start_powerSGD_iter) {
    if (f16 || prec != kStF32) {
      auto& slot = st->passthrough[bucket_index];
      if (!slot || !same_layout(*slot, numel, batched, prec, keys)) {
        auto pl = std::make_unique<BucketPlan>();
        pl->numel = numel;
        pl->batched = batched;
        pl->st = prec;
        pl->views = keys;
        if (batched)
          add_flat(pl->flat_all, 0, numel);
        else
          for (const ViewKey& k : pl->views) add_flat(pl->flat_all, k.offset, view_numel(k));
        powersgd_status u = upload(pl->flat_all, &pl->d_flat_all, s);
        if (u != POWERSGD_OK) return u;
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
        slot = std::move(pl);
      }
      BucketPlan& pl = *slot;
      const int nf = static_cast<int>(pl.flat_all.size());
      double all = 0;
      for (const FlatTile& f : pl.flat_all) all += static_cast<double>(f.len);
      if (prec != kStF32) {
        powersgd_status r = timed_launch(st, s, K_UNSCALE, all * 8.0, "16-bit cast", [&] {
          return launch_round_only(pl.d_flat_all, nf, bucket, prec, s);
        });
        if (r != POWERSGD_OK) return r;
        if (is_last) st->iteration += 1;
        return POWERSGD_OK;
      }
      powersgd_status r = timed_launch(st, s, K_UNSCALE, all * 2.0, "fp16 check", [&] {
        return launch_unscale_only(pl.d_flat_all, nf, bucket, inv_loss_scale, found_inf_dev,
                                   true, s);
      });
      if (r != POWERSGD_OK) return r;
      r = timed_launch(st, s, K_UNSCALE, all * 4.0, "fp16 unscale", [&] {
        return launch_unscale_only(pl.d_flat_all, nf, bucket, inv_loss_scale, found_inf_dev,
                                   false, s);
      });
      if (r != POWERSGD_OK) return r;
    }
    if (is_last) st->iteration += 1;
    return POWERSGD_OK;
  }

  // Plan lookup; a memorized bucket must keep its layout.
  auto it = st->buckets.find(bucket_index);
  if (it != st->buckets.end() && !same_layout(*it->second, numel, batched, prec, keys)) {
    if (ef || hp.warm_start)
      return fail(POWERSGD_ERR_LAYOUT_CHANGED,
                  "bucket " + std::to_string(bucket_index) + " was called with other views");
    st->buckets.erase(it);
    it = st->buckets.end();
  }
  if (it == st->buckets.end()) {
    auto pl = std::make_unique<BucketPlan>();
    powersgd_status b = build_plan(hp, numel, batched, prec, std::move(keys), *pl);
    if (b != POWERSGD_OK) return b;
    // an fp16 bucket's fp32 state keeps M' in two alternating places
    b = allocate_plan(*pl, ef, f16 && prec == kStF32, s);
    if (b != POWERSGD_OK) return b;
    it = st->buckets.emplace(bucket_index, std::move(pl)).first;
  }
  BucketPlan& pl = *it->second;
  pl.last_stream = s;
  const int R = pl.R;
  const int nt = static_cast<int>(pl.tensors.size());
  const bool aligned = (base % 16) == 0;
  const TensorDesc* td = aligned ? pl.d_td : pl.d_td_scalar;
  const double ce = static_cast<double>(pl.compressed_elems);
  const double ue = static_cast<double>(pl.uncompressed_elems);
  const double eps = hp.orthogonalization_epsilon;
  // vector ranks: the Gram partials come from pass 1, pass 2 orthogonalizes P itself
  // and pass 3 sums the pass-2 partials
  const bool fused = R <= kMaxFusedGramRank;
  const uint64_t bucket_key = static_cast<uint64_t>(bucket_index);
  powersgd_status r = POWERSGD_OK;
  // a call with error feedback keeps M' in E's place; it rebuilds the previous error
  // from M'_prev, P and the warm-start Q unless E's place holds the error itself
  const bool sm = ef;
  if (ef && pl.keeps_mprime() && !pl.w_holds_e && nt > 0 && !hp.warm_start) {
    // this call cannot rebuild (a fresh Q draw replaces the Q it would need): the error
    // itself goes into E's place first
    r = materialize_error(pl, nullptr, s);
    if (r != POWERSGD_OK) return r;
    const hipError_t e = launch_set_flag(pl.wflag, 1, s);
    if (e != hipSuccess) return hip_fail(e, "error flag");
    pl.w_holds_e = true;
  }

  if (nt > 0) {
    // Step 3.1: a fresh orthogonalized N(0, 1) draw when there is no warm Q.
    if (!hp.warm_start || !pl.q_ready) {
      const uint64_t epoch = hp.warm_start ? 0 : static_cast<uint64_t>(st->iteration);
      r = timed_launch(st, s, K_QINIT, 0.0, "q_init", [&] {
        return launch_qinit(R, pl.d_qinit, nt, pl.max_qcount, pl.Q, hp.random_seed,
                            bucket_key, epoch, prec, s);
      });
      if (r != POWERSGD_OK) return r;
      r = timed_launch(st, s, K_GRAM, 0.0, "Gram of Q", [&] {
        return launch_gram(R, pl.d_qgram_tiles, static_cast<int>(pl.qgram_tiles.size()),
                           pl.d_qjobs, pl.Q, nullptr, pl.gram, nullptr, prec, s);
      });
      if (r != POWERSGD_OK) return r;
      r = timed_launch(st, s, K_ORTH, 0.0, "orthogonalize Q", [&] {
        return launch_orth(R, pl.d_qjobs, nt, pl.max_qrows, pl.Q, pl.QT, pl.gram, pl.tmat, eps,
                           nullptr, prec, s);
      });
      if (r != POWERSGD_OK) return r;
    }
  }
  // Batched variant, step 1: the square matrix's padding past the bucket is zero.
  if (batched && nt > 0) {
    const int64_t side = pl.view_n[0];
    const int64_t pad = side * side - numel;
    if (pad > 0) {
      hipError_t e = launch_fill_zero(bucket, f16, numel, pad, s);
      if (e != hipSuccess) return hip_fail(e, "padding fill");
    }
  }
  // fp16 with M' kept in a single E's place: the inf check of every view comes first, so
  // that a step to be skipped writes nothing (pass 1 would overwrite M'_prev); with two
  // places pass 1 checks the bucket as it reads it.
  const bool precheck = f16 && sm && pl.wstride == 0;
  if (precheck) {
    const double all = static_cast<double>(pl.all_elems);
    r = timed_launch(st, s, K_UNSCALE, all * 2.0, "fp16 check", [&] {
      return launch_unscale_only(pl.d_flat_all, static_cast<int>(pl.flat_all.size()), bucket,
                                 inv_loss_scale, found_inf_dev, true, s);
    });
    if (r != POWERSGD_OK) return r;
  }
  // Pass 1 (+ fp16 inf check of every view when it did not run above).
  {
    Pass1Args a{};
    a.tiles = pl.d_tiles1;
    a.ntiles = static_cast<int32_t>(pl.tiles1.size());
    a.ftiles = pl.d_flat_unc;
    a.nftiles = precheck ? 0 : static_cast<int32_t>(pl.flat_unc.size());
    a.td = td;
    a.bucket = bucket;
    a.E = pl.E;
    a.Q = pl.Q;
    a.QT = pl.QT;
    a.P = fused ? pl.Praw : pl.P;
    a.Ppart = pl.Ppart;
    a.Pe = sm ? pl.P : nullptr;  // the kernels skip the rebuild while wflag is set
    a.wflag = sm ? pl.wflag : nullptr;
    a.widx = pl.widx;
    a.wstride = pl.wstride;
    a.gram = pl.gram;
    a.Eh = pl.Eh;
    a.Mh = pl.mprime16();
    a.inv_scale = inv_loss_scale;
    a.found_inf = found_inf_dev;
    const double bytes = ce * pass_bytes(K_PASS1, f16, ef, prec) + (f16 && !precheck ? ue * 2.0 : 0.0);
    r = timed_launch(st, s, K_PASS1, bytes, "pass 1",
                     [&] { return launch_pass1(R, f16, ef, prec, a, s); });
    if (r != POWERSGD_OK) return r;
  }
  if (nt > 0) {
    // Step 3.4 (the allreduce of P, step 3.3, is the identity on one rank).
    if (!pl.pgram_tiles.empty()) {
      r = timed_launch(st, s, K_GRAM, 0.0, "Gram of P", [&] {
        return launch_gram(R, pl.d_pgram_tiles, static_cast<int>(pl.pgram_tiles.size()),
                           pl.d_pjobs, pl.P, pl.Ppart, pl.gram, f16 ? found_inf_dev : nullptr,
                           prec, s);
      });
      if (r != POWERSGD_OK) return r;
    }
    if (!fused) {
      r = timed_launch(st, s, K_ORTH, 0.0, "orthogonalize P", [&] {
        return launch_orth(R, pl.d_pjobs, nt, pl.max_prows, pl.P, nullptr, pl.gram, pl.tmat,
                           eps, f16 ? found_inf_dev : nullptr, prec, s);
      });
      if (r != POWERSGD_OK) return r;
    }
    // Step 3.5 (step 3.6 is the identity); vector ranks orthogonalize P on the way in.
    Pass2Args a{};
    a.tiles = pl.d_tiles2;
    a.ntiles = static_cast<int32_t>(pl.tiles2.size());
    a.td = td;
    a.bucket = bucket;
    a.E = pl.E;
    a.P = fused ? pl.Praw : pl.P;
    a.Pout = pl.P;
    a.gram = pl.gram;
    a.eps = eps;
    a.Q = pl.Q;
    a.QT = pl.QT;
    a.partial = pl.partial;
    a.Mh = pl.mprime16();
    a.inv_scale = inv_loss_scale;
    a.found_inf = found_inf_dev;
    a.widx = pl.widx;
    a.wstride = pl.wstride;
    r = timed_launch(st, s, K_PASS2, ce * pass_bytes(K_PASS2, f16, ef, prec), "pass 2",
                     [&] {
                       return launch_pass2(R, f16, ef, prec, aligned && pl.all_wide, a, s);
                     });
    if (r != POWERSGD_OK) return r;
    if (!fused && !pl.tiles2r.empty()) {
      Pass2ReduceArgs b{};
      b.tiles = pl.d_tiles2r;
      b.ntiles = static_cast<int32_t>(pl.tiles2r.size());
      b.td = td;
      b.partial = pl.partial;
      b.Q = pl.Q;
      b.QT = pl.QT;
      b.found_inf = f16 ? found_inf_dev : nullptr;
      r = timed_launch(st, s, K_PASS2R, 0.0, "pass 2 reduce",
                       [&] { return launch_pass2_reduce(R, prec, b, s); });
      if (r != POWERSGD_OK) return r;
    }
  }
  {
    // Step 3.7 with the error update (+ fp16 unscale of the uncompressed views).
    Pass3Args a{};
    a.tiles = pl.d_tiles3;
    a.ntiles = static_cast<int32_t>(pl.tiles3.size());
    a.ftiles = pl.d_flat_unc;
    a.nftiles = static_cast<int32_t>(pl.flat_unc.size());
    a.td = td;
    a.bucket = bucket;
    a.E = pl.E;
    a.P = pl.P;
    a.Q = pl.Q;
    a.partial = pl.partial;  // vector ranks sum the pass-2 partials here
    a.Eh = pl.Eh;
    a.Mh = pl.mprime16();
    a.inv_scale = inv_loss_scale;
    a.found_inf = found_inf_dev;
    a.wflag = sm ? pl.wflag : nullptr;  // cleared by the pass once the step runs
    a.widx = pl.widx;                   // switched by the pass once the step runs
    a.wstride = pl.wstride;
    const double bytes = ce * pass_bytes(K_PASS3, f16, ef, prec) +
                         (f16 ? ue * 4.0 : (prec != kStF32 ? ue * 8.0 : 0.0));
    r = timed_launch(st, s, K_PASS3, bytes, "pass 3",
                     [&] { return launch_pass3(R, f16, ef, prec, a, s); });
    if (r != POWERSGD_OK) return r;
  }
  pl.q_ready = hp.warm_start != 0;
  if (sm && nt > 0) pl.w_holds_e = false;

  st->numel_in += pl.all_elems;
  st->numel_comm += pl.comm_elems;
  if (is_last) {
    if (hp.compression_stats_logging_frequency > 0 && st->iteration >= st->next_log_iteration) {
      std::fprintf(stderr,
                   "powersgd: iteration %lld, compression rate %.3f (%lld elements in, "
                   "%lld communicated)\n",
                   static_cast<long long>(st->iteration),
                   st->numel_comm > 0 ? static_cast<double>(st->numel_in) / st->numel_comm : 0.0,
                   static_cast<long long>(st->numel_in), static_cast<long long>(st->numel_comm));
      st->next_log_iteration = st->iteration + hp.compression_stats_logging_frequency;
    }
    st->iteration += 1;
  }
  return POWERSGD_OK;
}


}  // namespace

powersgd_status powersgd_compress_bucket(powersgd_state* st, int64_t bucket_index,
                                         int32_t is_last, void* bucket,
                                         powersgd_dtype dtype, int64_t numel,
                                         const powersgd_view* views, int32_t nviews,
                                         float inv_loss_scale, int32_t* found_inf_dev,
                                         void* stream) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (numel < 0) return fail(POWERSGD_ERR_INVALID_ARG, "numel < 0");
  if (nviews < 0) return fail(POWERSGD_ERR_INVALID_ARG, "nviews < 0");
  if (nviews > 0 && !views) return fail(POWERSGD_ERR_INVALID_ARG, "views is NULL");
  if (numel > 0 && !bucket) return fail(POWERSGD_ERR_INVALID_ARG, "bucket is NULL");
  if (dtype != POWERSGD_F32 && dtype != POWERSGD_F16)
    return fail(POWERSGD_ERR_INVALID_ARG, "unknown dtype");
  const bool f16 = dtype == POWERSGD_F16;
  if (f16 && !found_inf_dev)
    return fail(POWERSGD_ERR_INVALID_ARG, "fp16 buckets need found_inf_dev");
  if (f16 && !std::isfinite(inv_loss_scale))
    return fail(POWERSGD_ERR_INVALID_ARG, "inv_loss_scale must be finite");
  std::vector<ViewKey> keys;
  powersgd_status vs = validate_views(views, nviews, numel, keys);
  if (vs != POWERSGD_OK) return vs;
  return run_call(st, bucket_index, is_last, bucket, f16, numel, false, kStF32, keys,
                  inv_loss_scale, found_inf_dev, stream);
}

powersgd_status powersgd_compress_bucket_wrapped(powersgd_state* st, int64_t bucket_index,
                                                 int32_t is_last, float* bucket,
                                                 powersgd_dtype compute_dtype, int64_t numel,
                                                 const powersgd_view* views, int32_t nviews,
                                                 void* stream) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (numel < 0) return fail(POWERSGD_ERR_INVALID_ARG, "numel < 0");
  if (nviews < 0) return fail(POWERSGD_ERR_INVALID_ARG, "nviews < 0");
  if (nviews > 0 && !views) return fail(POWERSGD_ERR_INVALID_ARG, "views is NULL");
  if (numel > 0 && !bucket) return fail(POWERSGD_ERR_INVALID_ARG, "bucket is NULL");
  int prec = kStF32;
  if (compute_dtype == POWERSGD_F16)
    prec = kStF16;
  else if (compute_dtype == POWERSGD_BF16)
    prec = kStBF16;
  else
    return fail(POWERSGD_ERR_INVALID_ARG, "compute_dtype must be F16 or BF16");
  std::vector<ViewKey> keys;
  powersgd_status vs = validate_views(views, nviews, numel, keys);
  if (vs != POWERSGD_OK) return vs;
  return run_call(st, bucket_index, is_last, bucket, false, numel, false, prec, keys, 1.0f,
                  nullptr, stream);
}

int64_t powersgd_batched_side(int64_t numel) { return batched_side(numel); }

powersgd_status powersgd_compress_bucket_batched_wrapped(powersgd_state* st, int64_t bucket_index,
                                                         int32_t is_last, float* bucket,
                                                         powersgd_dtype compute_dtype,
                                                         int64_t numel, int64_t capacity,
                                                         void* stream) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (numel < 0) return fail(POWERSGD_ERR_INVALID_ARG, "numel < 0");
  if (numel > 0 && !bucket) return fail(POWERSGD_ERR_INVALID_ARG, "bucket is NULL");
  int prec = kStF32;
  if (compute_dtype == POWERSGD_F16)
    prec = kStF16;
  else if (compute_dtype == POWERSGD_BF16)
    prec = kStBF16;
  else
    return fail(POWERSGD_ERR_INVALID_ARG, "compute_dtype must be F16 or BF16");
  const int64_t side = batched_side(numel);
  if (side > kMaxMatrixDim) return fail(POWERSGD_ERR_UNSUPPORTED, "bucket too large for the batched view");
  if (capacity < side * side)
    return fail(POWERSGD_ERR_INVALID_ARG,
                "capacity " + std::to_string(capacity) + " is below the padded square of " +
                    std::to_string(side * side) + " elements");
  std::vector<ViewKey> keys;
  if (numel > 0) keys.push_back(ViewKey{0, {side, side}});
  return run_call(st, bucket_index, is_last, bucket, false, numel, true, prec, keys, 1.0f,
                  nullptr, stream);
}

powersgd_status powersgd_compress_bucket_batched(powersgd_state* st, int64_t bucket_index,
                                                 int32_t is_last, void* bucket,
                                                 powersgd_dtype dtype, int64_t numel,
                                                 int64_t capacity, float inv_loss_scale,
                                                 int32_t* found_inf_dev, void* stream) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (numel < 0) return fail(POWERSGD_ERR_INVALID_ARG, "numel < 0");
  if (numel > 0 && !bucket) return fail(POWERSGD_ERR_INVALID_ARG, "bucket is NULL");
  if (dtype != POWERSGD_F32 && dtype != POWERSGD_F16)
    return fail(POWERSGD_ERR_INVALID_ARG, "unknown dtype");
  const bool f16 = dtype == POWERSGD_F16;
  if (f16 && !found_inf_dev)
    return fail(POWERSGD_ERR_INVALID_ARG, "fp16 buckets need found_inf_dev");
  if (f16 && !std::isfinite(inv_loss_scale))
    return fail(POWERSGD_ERR_INVALID_ARG, "inv_loss_scale must be finite");
  const int64_t side = batched_side(numel);
  if (side > kMaxMatrixDim) return fail(POWERSGD_ERR_UNSUPPORTED, "bucket too large for the batched view");
  if (capacity < side * side)
    return fail(POWERSGD_ERR_INVALID_ARG,
                "capacity " + std::to_string(capacity) + " is below the padded square of " +
                    std::to_string(side * side) + " elements");
  std::vector<ViewKey> keys;
  if (numel > 0) keys.push_back(ViewKey{0, {side, side}});
  return run_call(st, bucket_index, is_last, bucket, f16, numel, true, kStF32, keys,
                  inv_loss_scale, found_inf_dev, stream);
}

powersgd_status powersgd_classify_view(const powersgd_hparams* hp, const powersgd_view* view,
                                       int32_t* compress, int64_t* n, int64_t* m,
                                       int32_t* rank) {
  if (!hp || !view) return fail(POWERSGD_ERR_INVALID_ARG, "NULL argument");
  if (view->ndim < 0 || view->ndim > POWERSGD_MAX_NDIM)
    return fail(POWERSGD_ERR_INVALID_ARG, "ndim out of range");
  int64_t size = 1;
  for (int64_t d = 0; d < view->ndim; ++d) {
    if (view->shape[d] < 0) return fail(POWERSGD_ERR_INVALID_ARG, "negative dimension");
    if (view->shape[d] > 0 && size > INT64_MAX / view->shape[d])
      return fail(POWERSGD_ERR_INVALID_ARG, "size overflows");
    size *= view->shape[d];
  }
  int64_t rows = 0, cols = 0, rk = 0;
  bool comp = false;
  if (view->ndim >= 2) {
    rows = view->shape[0];
    cols = 1;
    for (int64_t d = 1; d < view->ndim; ++d) cols *= view->shape[d];
    rk = std::min<int64_t>(hp->matrix_approximation_rank, std::min(rows, cols));
    comp = rk >= 1 && should_compress(rows, cols, rk, hp->min_compression_rate);
  }
  if (compress) *compress = comp ? 1 : 0;
  if (n) *n = view->ndim >= 2 ? rows : 0;
  if (m) *m = view->ndim >= 2 ? cols : 0;
  if (rank) *rank = comp ? static_cast<int32_t>(rk) : 0;
  return POWERSGD_OK;
}

powersgd_status powersgd_get_decisions(powersgd_state* st, int64_t bucket_index, uint8_t* out,
                                       int32_t nviews) {
  if (!st || !out) return fail(POWERSGD_ERR_INVALID_ARG, "NULL argument");
  auto it = st->buckets.find(bucket_index);
  if (it == st->buckets.end()) return fail(POWERSGD_ERR_NOT_FOUND, "bucket never compressed");
  const BucketPlan& pl = *it->second;
  if (nviews != static_cast<int32_t>(pl.decision.size()))
    return fail(POWERSGD_ERR_INVALID_ARG, "nviews does not match the bucket");
  std::memcpy(out, pl.decision.data(), pl.decision.size());
  return POWERSGD_OK;
}

powersgd_status powersgd_get_view_info(powersgd_state* st, int64_t bucket_index, int32_t view,
                                       int64_t* n, int64_t* m, int32_t* rank) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  auto it = st->buckets.find(bucket_index);
  if (it == st->buckets.end()) return fail(POWERSGD_ERR_NOT_FOUND, "bucket never compressed");
  const BucketPlan& pl = *it->second;
  if (view < 0 || view >= static_cast<int32_t>(pl.views.size()))
    return fail(POWERSGD_ERR_INVALID_ARG, "view out of range");
  if (n) *n = pl.view_n[view];
  if (m) *m = pl.view_m[view];
  if (rank) *rank = pl.view_rank[view];
  return POWERSGD_OK;
}

static powersgd_status find_tensor(powersgd_state* st, int64_t bucket_index, int32_t view,
                                   BucketPlan** plp, const TensorDesc** dp) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  auto it = st->buckets.find(bucket_index);
  if (it == st->buckets.end()) return fail(POWERSGD_ERR_NOT_FOUND, "bucket never compressed");
  BucketPlan& pl = *it->second;
  if (view < 0 || view >= static_cast<int32_t>(pl.views.size()))
    return fail(POWERSGD_ERR_INVALID_ARG, "view out of range");
  const int32_t t = pl.view_tensor[view];
  if (t < 0) return fail(POWERSGD_ERR_NOT_FOUND, "view is not compressed");
  *plp = &pl;
  *dp = &pl.tensors[t];
  return POWERSGD_OK;
}

powersgd_status powersgd_copy_factors(powersgd_state* st, int64_t bucket_index, int32_t view,
                                      float* p_dev, float* q_dev, void* stream) {
  BucketPlan* pl = nullptr;
  const TensorDesc* d = nullptr;
  powersgd_status r = find_tensor(st, bucket_index, view, &pl, &d);
  if (r != POWERSGD_OK) return r;
  HipDeviceGuard guard(st->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t R = pl->R;
  // P and Q are stored with row stride R; copy the first `rank` columns of each row.
  if (p_dev) {
    hipError_t e = hipMemcpy2DAsync(p_dev, d->rank * sizeof(float), pl->P + d->poff,
                                    R * sizeof(float), d->rank * sizeof(float), d->n,
                                    hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "copy of P");
  }
  if (q_dev) {
    hipError_t e = hipMemcpy2DAsync(q_dev, d->rank * sizeof(float), pl->Q + d->qoff,
                                    R * sizeof(float), d->rank * sizeof(float), d->m,
                                    hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "copy of Q");
  }
  return POWERSGD_OK;
}

powersgd_status powersgd_copy_error(powersgd_state* st, int64_t bucket_index, int32_t view,
                                    float* e_dev, void* stream) {
  BucketPlan* pl = nullptr;
  const TensorDesc* d = nullptr;
  powersgd_status r = find_tensor(st, bucket_index, view, &pl, &d);
  if (r != POWERSGD_OK) return r;
  if (!pl->E && !pl->Eh) return fail(POWERSGD_ERR_NOT_FOUND, "error feedback is off");
  if (!e_dev) return fail(POWERSGD_ERR_INVALID_ARG, "e_dev is NULL");
  HipDeviceGuard guard(st->device);
  if (pl->Eh && pl->w_holds_e) {
    // a 16-bit state holding the error itself: its values widened to fp32
    hipError_t e = launch_widen16(pl->Eh + d->eoff, e_dev, static_cast<int64_t>(d->n) * d->m,
                                  pl->st, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy of E");
    return POWERSGD_OK;
  }
  const float* src = nullptr;
  r = error_source(*pl, static_cast<hipStream_t>(stream), &src);
  if (r != POWERSGD_OK) return r;
  hipError_t e = hipMemcpyAsync(e_dev, src + d->eoff,
                                static_cast<size_t>(d->n) * d->m * sizeof(float),
                                hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy of E");
  return POWERSGD_OK;
}

powersgd_status powersgd_get_factors(powersgd_state* st, int64_t bucket_index, int32_t view,
                                     const float** P_dev, const float** Q_dev, int64_t* n,
                                     int64_t* m, int32_t* r) {
  BucketPlan* pl = nullptr;
  const TensorDesc* d = nullptr;
  powersgd_status rs = find_tensor(st, bucket_index, view, &pl, &d);
  if (rs != POWERSGD_OK) return rs;
  HipDeviceGuard guard(st->device);
  if (!guard.ok) return fail(POWERSGD_ERR_HIP, "hipSetDevice failed");
  if (!pl->intro_PQ) {
    // one compact n x rank P and m x rank Q per tensor, in tensor order
    std::vector<int64_t> off;
    int64_t total = 0;
    for (const TensorDesc& t : pl->tensors) {
      off.push_back(total);
      total += (static_cast<int64_t>(t.n) + t.m) * t.rank;
    }
    void* p = nullptr;
    if (hipMalloc(&p, std::max<int64_t>(total, 1) * sizeof(float)) != hipSuccess)
      return fail(POWERSGD_ERR_OOM, "allocation of the factor copies failed");
    pl->intro_PQ = static_cast<float*>(p);
    pl->intro_off = std::move(off);
  }
  const int32_t t = pl->view_tensor[view];
  float* pc = pl->intro_PQ + pl->intro_off[t];
  float* qc = pc + static_cast<int64_t>(d->n) * d->rank;
  hipStream_t s = pl->last_stream;
  const size_t R = pl->R;
  hipError_t e = hipMemcpy2DAsync(pc, d->rank * sizeof(float), pl->P + d->poff,
                                  R * sizeof(float), d->rank * sizeof(float), d->n,
                                  hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpy2DAsync(qc, d->rank * sizeof(float), pl->Q + d->qoff, R * sizeof(float),
                         d->rank * sizeof(float), d->m, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "copy of the factors");
  if (P_dev) *P_dev = pc;
  if (Q_dev) *Q_dev = qc;
  if (n) *n = d->n;
  if (m) *m = d->m;
  if (r) *r = d->rank;
  return POWERSGD_OK;
}

powersgd_status powersgd_get_error(powersgd_state* st, int64_t bucket_index, const float** E_dev) {
  if (!st || !E_dev) return fail(POWERSGD_ERR_INVALID_ARG, "NULL argument");
  auto it = st->buckets.find(bucket_index);
  if (it == st->buckets.end()) return fail(POWERSGD_ERR_NOT_FOUND, "bucket never compressed");
  BucketPlan& pl = *it->second;
  if (!pl.E && !pl.Eh) return fail(POWERSGD_ERR_NOT_FOUND, "error feedback is off");
  HipDeviceGuard guard(st->device);
  if (!guard.ok) return fail(POWERSGD_ERR_HIP, "hipSetDevice failed");
  // the batched variant's bucket is its s x s padded matrix
  const int64_t len = pl.batched ? (pl.tensors.empty() ? 0 : view_numel(pl.views[0]))
                                 : pl.numel;
  if (!pl.intro_E) {
    void* p = nullptr;
    if (hipMalloc(&p, std::max<int64_t>(len, 1) * sizeof(float)) != hipSuccess)
      return fail(POWERSGD_ERR_OOM, "allocation of the bucket-shaped error failed");
    pl.intro_E = static_cast<float*>(p);
  }
  hipStream_t s = pl.last_stream;
  const float* src = nullptr;
  // a 16-bit state holding the error itself is widened; otherwise the binary32 error
  const bool widen = pl.Eh && pl.w_holds_e;
  if (!widen) {
    powersgd_status rs = error_source(pl, s, &src);
    if (rs != POWERSGD_OK) return rs;
  }
  hipError_t e = launch_fill_zero(pl.intro_E, false, 0, len, s);
  for (const TensorDesc& d : pl.tensors) {
    if (e != hipSuccess) break;
    const int64_t cnt = static_cast<int64_t>(d.n) * d.m;
    if (widen)
      e = launch_widen16(pl.Eh + d.eoff, pl.intro_E + d.boff, cnt, pl.st, s);
    else
      e = hipMemcpyAsync(pl.intro_E + d.boff, src + d.eoff, cnt * sizeof(float),
                         hipMemcpyDeviceToDevice, s);
  }
  if (e != hipSuccess) return hip_fail(e, "fill of the bucket-shaped error");
  *E_dev = pl.intro_E;
  return POWERSGD_OK;
}

powersgd_status powersgd_draw_q0(uint64_t random_seed, int64_t bucket_index, int32_t view,
                                 uint64_t epoch, int64_t m, int32_t rank, float* out_dev,
                                 uint64_t* words_dev, void* stream) {
  if (m < 0) return fail(POWERSGD_ERR_INVALID_ARG, "m < 0");
  if (rank < 1) return fail(POWERSGD_ERR_INVALID_ARG, "rank < 1");
  if (view < 0) return fail(POWERSGD_ERR_INVALID_ARG, "view < 0");
  if (rank > POWERSGD_MAX_RANK) return fail(POWERSGD_ERR_UNSUPPORTED, "rank above 32");
  if (m > kMaxMatrixDim) return fail(POWERSGD_ERR_UNSUPPORTED, "m above 2^31 - 65537");
  if (m > 0 && !out_dev) return fail(POWERSGD_ERR_INVALID_ARG, "out_dev is NULL");
  hipError_t e = launch_qdraw(m, rank, view, out_dev, words_dev, random_seed,
                              static_cast<uint64_t>(bucket_index), epoch,
                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "initial Q draw");
  return POWERSGD_OK;
}

powersgd_status powersgd_get_stats(powersgd_state* st, int64_t* iteration, int64_t* numel_in,
                                   int64_t* numel_comm) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (iteration) *iteration = st->iteration;
  if (numel_in) *numel_in = st->numel_in;
  if (numel_comm) *numel_comm = st->numel_comm;
  return POWERSGD_OK;
}

// --- state snapshot --------------------------------------------------------------
// The byte format is the one include/powersgd.h defines (version 1).

extern "C++" {
namespace {

static_assert(__BYTE_ORDER__ == __ORDER_LITTLE_ENDIAN__, "the snapshot format is little-endian");

constexpr char kSnapMagic[8] = {'P', 'S', 'G', 'D', 'S', 'N', 'A', 'P'};
constexpr uint32_t kSnapVersion = 1;

// Appends fields at `pos`; with a NULL base it only measures.
struct SnapWriter {
  uint8_t* base = nullptr;
  int64_t pos = 0;
  template <class T>
  void put(T v) {
    if (base) std::memcpy(base + pos, &v, sizeof(T));
    pos += static_cast<int64_t>(sizeof(T));
  }
  uint8_t* take(int64_t bytes) {
    uint8_t* at = base ? base + pos : nullptr;
    pos += bytes;
    return at;
  }
};

// Reads fields from [base, base + size); every read is checked against the end.
struct SnapReader {
  const uint8_t* base;
  int64_t size;
  int64_t pos = 0;
  template <class T>
  bool get(T& v) {
    if (size - pos < static_cast<int64_t>(sizeof(T))) return false;
    std::memcpy(&v, base + pos, sizeof(T));
    pos += static_cast<int64_t>(sizeof(T));
    return true;
  }
  const uint8_t* take(int64_t bytes) {
    if (bytes < 0 || size - pos < bytes) return nullptr;
    const uint8_t* at = base + pos;
    pos += bytes;
    return at;
  }
};

// 16-bit state values on the host (snapshots): bfloat16 rounded to nearest even from
// the binary32 pattern (as the kernels do), binary16 through the compiler's _Float16.
uint16_t host_to_h16(float x, int prec) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if (prec == kStBF16) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
  const _Float16 h = static_cast<_Float16>(x);
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

float host_from_h16(uint16_t h, int prec) {
  float f;
  if (prec == kStBF16) {
    const uint32_t u = static_cast<uint32_t>(h) << 16;
    std::memcpy(&f, &u, 4);
    return f;
  }
  _Float16 v;
  std::memcpy(&v, &h, 2);
  return static_cast<float>(v);
}

uint32_t snap_flags(const powersgd_hparams& hp) {
  return (hp.use_error_feedback ? 1u : 0u) | (hp.warm_start ? 2u : 0u);
}

bool snap_has_q(const powersgd_hparams& hp, const BucketPlan& pl) {
  return hp.warm_start && pl.q_ready && !pl.tensors.empty();
}

// One contiguous transfer between device memory and (pageable) host memory.
struct CopySeg {
  void* dev;
  uint8_t* host;
  int64_t bytes;
};

// Runs the transfers through two pinned staging buffers on stream s: the DMA of one
// buffer overlaps the host memcpy of the other (pageable transfers run at a fraction
// of the link rate). Returns after every transfer has completed.
powersgd_status staged_copy(const std::vector<CopySeg>& segs, bool to_host, hipStream_t s) {
  constexpr int64_t kStageBytes = int64_t{16} << 20;
  int64_t total = 0;
  for (const CopySeg& c : segs) total += c.bytes;
  if (total == 0) return POWERSGD_OK;
  const int64_t cap = std::min(total, kStageBytes);
  uint8_t* pin[2] = {nullptr, nullptr};
  hipEvent_t ev[2] = {nullptr, nullptr};
  struct Piece {
    uint8_t* host;
    int64_t at, bytes;
  };
  std::vector<Piece> pending[2];
  bool busy[2] = {false, false};
  powersgd_status r = POWERSGD_OK;
  auto check = [&](hipError_t e, const char* what) {
    if (e != hipSuccess && r == POWERSGD_OK) r = hip_fail(e, what);
    return r == POWERSGD_OK;
  };
  // waits for buffer b's transfers; device-to-host pieces are then copied out
  auto drain = [&](int b) {
    if (!busy[b]) return;
    busy[b] = false;
    if (!check(hipEventSynchronize(ev[b]), "staged copy")) return;
    for (const Piece& pc : pending[b]) std::memcpy(pc.host, pin[b] + pc.at, pc.bytes);
    pending[b].clear();
  };
  for (int b = 0; b < 2 && r == POWERSGD_OK; ++b) {
    check(hipHostMalloc(reinterpret_cast<void**>(&pin[b]), cap, hipHostMallocDefault),
          "hipHostMalloc of the staging buffer");
    if (r == POWERSGD_OK) check(hipEventCreateWithFlags(&ev[b], hipEventDisableTiming), "hipEventCreate");
  }
  int b = 0;
  int64_t fill = 0;
  for (const CopySeg& c : segs) {
    int64_t done = 0;
    while (done < c.bytes && r == POWERSGD_OK) {
      const int64_t n = std::min(c.bytes - done, cap - fill);
      uint8_t* dev = static_cast<uint8_t*>(c.dev) + done;
      if (to_host) {
        check(hipMemcpyAsync(pin[b] + fill, dev, n, hipMemcpyDeviceToHost, s), "staged copy");
        pending[b].push_back(Piece{c.host + done, fill, n});
      } else {
        std::memcpy(pin[b] + fill, c.host + done, n);
        check(hipMemcpyAsync(dev, pin[b] + fill, n, hipMemcpyHostToDevice, s), "staged copy");
      }
      done += n;
      fill += n;
      if (fill == cap) {
        check(hipEventRecord(ev[b], s), "hipEventRecord");
        busy[b] = true;
        b ^= 1;
        drain(b);
        fill = 0;
      }
    }
  }
  if (fill > 0 && r == POWERSGD_OK) {
    check(hipEventRecord(ev[b], s), "hipEventRecord");
    busy[b] = true;
  }
  // every enqueued transfer ends before the staging buffers are freed, also on error
  (void)hipStreamSynchronize(s);
  for (int k = 0; k < 2; ++k) {
    if (r == POWERSGD_OK) drain(k);
    if (ev[k]) (void)hipEventDestroy(ev[k]);
    if (pin[k]) (void)hipHostFree(pin[k]);
  }
  return r;
}

// Device-to-host work of an export: the transfers, and for every warm-start Q the
// whole strided Q buffer of its bucket, compacted into the snapshot afterwards.
struct ExportCopies {
  std::vector<CopySeg> segs;
  std::vector<std::vector<float>> qbufs;  // per bucket with a Q: its Q buffer (row stride R)
  struct QPiece {
    size_t qbuf;
    int64_t qoff;
    int32_t m, rank, R;
    uint8_t* dst;
  };
  std::vector<QPiece> qpieces;
  std::vector<std::vector<uint16_t>> ebufs;  // per 16-bit bucket: its E buffer
  struct EPiece {
    size_t ebuf;
    int64_t eoff, count;
    int prec;
    uint8_t* dst;
  };
  std::vector<EPiece> epieces;
};

// Writes (or measures, with w.base NULL) the snapshot; with `copies` it lists the
// E and Q transfers instead of writing their bytes.
void write_snapshot(const powersgd_state* st, SnapWriter& w, ExportCopies* copies) {
  const powersgd_hparams& hp = st->hp;
  const bool ef = hp.use_error_feedback != 0;
  for (char c : kSnapMagic) w.put(c);
  w.put<uint32_t>(kSnapVersion);
  w.put<uint32_t>(snap_flags(hp));
  w.put<int32_t>(hp.matrix_approximation_rank);
  w.put<uint32_t>(0);
  w.put<double>(hp.min_compression_rate);
  w.put<uint64_t>(hp.random_seed);
  w.put<int64_t>(st->iteration);
  w.put<int64_t>(st->numel_in);
  w.put<int64_t>(st->numel_comm);
  w.put<int64_t>(st->next_log_iteration);
  w.put<int64_t>(static_cast<int64_t>(st->buckets.size()));
  for (const auto& kv : st->buckets) {  // std::map: ascending bucket index
    const BucketPlan& pl = *kv.second;
    const bool has_q = snap_has_q(hp, pl);
    w.put<int64_t>(kv.first);
    w.put<int64_t>(pl.numel);
    w.put<uint32_t>((pl.batched ? 1u : 0u) | (static_cast<uint32_t>(pl.st) << 8));
    w.put<uint32_t>(has_q ? 1u : 0u);
    w.put<int64_t>(static_cast<int64_t>(pl.views.size()));
    for (const ViewKey& k : pl.views) {
      w.put<int64_t>(k.offset);
      w.put<int64_t>(static_cast<int64_t>(k.shape.size()));
      for (int64_t d : k.shape) w.put<int64_t>(d);
    }
    size_t qbuf = 0, ebuf = 0;
    // a 16-bit E's place holding the error itself goes over in 16 bits and is widened on
    // the host; any other error comes from binary32 memory (E's place, or the error the
    // export materialized first)
    const bool e16 = pl.st != kStF32 && pl.w_holds_e;
    if (copies && ef && e16 && pl.e_floats > 0) {
      copies->ebufs.emplace_back(static_cast<size_t>(pl.e_floats));
      ebuf = copies->ebufs.size() - 1;
      copies->segs.push_back(CopySeg{pl.Eh, reinterpret_cast<uint8_t*>(copies->ebufs[ebuf].data()),
                                     pl.e_floats * 2});
    }
    if (copies && has_q) {
      copies->qbufs.emplace_back(static_cast<size_t>(pl.q_floats));
      qbuf = copies->qbufs.size() - 1;
      copies->segs.push_back(CopySeg{pl.Q, reinterpret_cast<uint8_t*>(copies->qbufs[qbuf].data()),
                                     pl.q_floats * 4});
    }
    for (size_t v = 0; v < pl.views.size(); ++v) {
      const int32_t t = pl.view_tensor[v];
      if (t < 0) continue;
      const TensorDesc& d = pl.tensors[t];
      if (ef) {
        const int64_t bytes = static_cast<int64_t>(d.n) * d.m * 4;
        uint8_t* dst = w.take(bytes);
        if (copies && bytes > 0) {
          if (e16)  // widened to binary32 after the transfer
            copies->epieces.push_back(
                ExportCopies::EPiece{ebuf, d.eoff, static_cast<int64_t>(d.n) * d.m, pl.st, dst});
          else
            copies->segs.push_back(
                CopySeg{(pl.w_holds_e && pl.wstride == 0 ? pl.E : pl.Emat) + d.eoff, dst,
                        bytes});
        }
      }
      if (has_q) {
        uint8_t* dst = w.take(static_cast<int64_t>(d.m) * d.rank * 4);
        if (copies)
          copies->qpieces.push_back(ExportCopies::QPiece{qbuf, d.qoff, d.m, d.rank, pl.R, dst});
      }
    }
  }
}

// One bucket record of a snapshot being imported: its new plan and where its E and Q
// blocks sit in the snapshot, per tensor.
struct SnapBucket {
  int64_t index = 0;
  bool has_q = false;
  std::unique_ptr<BucketPlan> plan;
  std::vector<const uint8_t*> e_src, q_src;
};

powersgd_status snap_bad(const std::string& what) {
  return fail(POWERSGD_ERR_INVALID_ARG, "snapshot: " + what);
}

powersgd_status read_bucket(const powersgd_hparams& hp, SnapReader& rd, int64_t prev_index,
                            SnapBucket& out) {
  int64_t numel = 0, nviews = 0;
  uint32_t variant = 0, has_q = 0;
  if (!rd.get(out.index) || !rd.get(numel) || !rd.get(variant) || !rd.get(has_q) ||
      !rd.get(nviews))
    return snap_bad("truncated bucket record");
  if (out.index <= prev_index) return snap_bad("bucket indices not strictly ascending");
  const uint32_t batched = variant & 1u;
  const int prec = static_cast<int>((variant >> 8) & 3u);
  if (numel < 0 || nviews < 0 || (variant & ~0x301u) != 0 || prec == 3 || has_q > 1)
    return snap_bad("bad field in the record of bucket " + std::to_string(out.index));
  if (has_q && !hp.warm_start) return snap_bad("warm-start Q without warm start");
  // every view record takes at least 16 bytes
  if (nviews > (rd.size - rd.pos) / 16) return snap_bad("truncated view records");
  std::vector<powersgd_view> views(static_cast<size_t>(nviews));
  for (powersgd_view& pv : views) {
    std::memset(&pv, 0, sizeof(pv));
    int64_t ndim = 0;  // an i64 in the snapshot, an int32 in powersgd_view
    if (!rd.get(pv.offset) || !rd.get(ndim)) return snap_bad("truncated view record");
    if (ndim < 0 || ndim > POWERSGD_MAX_NDIM) return snap_bad("view ndim out of range");
    pv.ndim = static_cast<int32_t>(ndim);
    for (int64_t d = 0; d < pv.ndim; ++d)
      if (!rd.get(pv.shape[d])) return snap_bad("truncated view shape");
  }
  std::vector<ViewKey> keys;
  if (batched) {
    const int64_t side = batched_side(numel);
    if (side > kMaxMatrixDim) return fail(POWERSGD_ERR_UNSUPPORTED, "snapshot: batched bucket too large");
    const bool ok = numel == 0 ? nviews == 0
                               : nviews == 1 && views[0].offset == 0 && views[0].ndim == 2 &&
                                     views[0].shape[0] == side && views[0].shape[1] == side;
    if (!ok) return snap_bad("batched bucket " + std::to_string(out.index) + " is not one s x s view");
    if (numel > 0) keys.push_back(ViewKey{0, {side, side}});
  } else {
    powersgd_status vs = validate_views(views.data(), static_cast<int32_t>(nviews), numel, keys);
    if (vs != POWERSGD_OK) return vs;
    if (nviews > INT32_MAX) return snap_bad("too many views");
  }
  out.plan = std::make_unique<BucketPlan>();
  powersgd_status b = build_plan(hp, numel, batched != 0, prec, std::move(keys), *out.plan);
  if (b != POWERSGD_OK) return b;
  BucketPlan& pl = *out.plan;
  if (has_q && pl.tensors.empty()) return snap_bad("warm-start Q on a bucket with no compressed view");
  out.has_q = has_q != 0;
  out.e_src.assign(pl.tensors.size(), nullptr);
  out.q_src.assign(pl.tensors.size(), nullptr);
  for (size_t v = 0; v < pl.views.size(); ++v) {
    const int32_t t = pl.view_tensor[v];
    if (t < 0) continue;
    const TensorDesc& d = pl.tensors[t];
    if (hp.use_error_feedback) {
      out.e_src[t] = rd.take(static_cast<int64_t>(d.n) * d.m * 4);
      if (!out.e_src[t]) return snap_bad("truncated error memory");
    }
    if (has_q) {
      out.q_src[t] = rd.take(static_cast<int64_t>(d.m) * d.rank * 4);
      if (!out.q_src[t]) return snap_bad("truncated warm-start Q");
    }
  }
  return POWERSGD_OK;
}

// Allocates a parsed bucket's device memory and lists the uploads of its E, its Q
// buffer (row stride R) and, for matrix-core ranks, Q transposed; the Q buffers are
// assembled on the host in `keep`, which must outlive the transfers.
powersgd_status upload_bucket(const powersgd_hparams& hp, SnapBucket& sb, hipStream_t s,
                              std::vector<CopySeg>& segs,
                              std::list<std::vector<float>>& keep,
                              std::list<std::vector<uint16_t>>& keep16) {
  BucketPlan& pl = *sb.plan;
  // one E's place (a later fp16 call then checks the bucket before pass 1)
  powersgd_status r = allocate_plan(pl, hp.use_error_feedback != 0, false, s);
  if (r != POWERSGD_OK) return r;
  const int prec = pl.st;
  std::vector<uint16_t>* eh = nullptr;  // a 16-bit E, rounded from the snapshot's binary32
  if (prec != kStF32 && pl.Eh) {
    keep16.emplace_back(static_cast<size_t>(pl.e_floats), uint16_t{0});
    eh = &keep16.back();
  }
  std::vector<float>* q = nullptr;
  std::vector<float>* qt = nullptr;
  if (sb.has_q) {
    // columns past each tensor's rank, and Q^T's rows past it and columns past m, stay zero
    keep.emplace_back(static_cast<size_t>(pl.q_floats), 0.f);
    q = &keep.back();
    if (pl.QT) {
      keep.emplace_back(static_cast<size_t>(pl.qt_floats), 0.f);
      qt = &keep.back();
    }
  }
  for (size_t t = 0; t < pl.tensors.size(); ++t) {
    const TensorDesc& d = pl.tensors[t];
    const int64_t ne = static_cast<int64_t>(d.n) * d.m;
    if (sb.e_src[t] && ne > 0) {
      if (eh) {
        for (int64_t i = 0; i < ne; ++i) {
          float v;
          std::memcpy(&v, sb.e_src[t] + i * 4, 4);
          (*eh)[static_cast<size_t>(d.eoff + i)] = host_to_h16(v, prec);
        }
      } else {
        segs.push_back(CopySeg{pl.E + d.eoff, const_cast<uint8_t*>(sb.e_src[t]), ne * 4});
      }
    }
    if (!q || !sb.q_src[t]) continue;
    for (int32_t j = 0; j < d.m; ++j)
      for (int32_t k = 0; k < d.rank; ++k) {
        float v;
        std::memcpy(&v, sb.q_src[t] + (static_cast<size_t>(j) * d.rank + k) * 4, 4);
        if (prec != kStF32) v = host_from_h16(host_to_h16(v, prec), prec);
        (*q)[static_cast<size_t>(d.qoff) + static_cast<size_t>(j) * pl.R + k] = v;
        if (qt && d.qtoff >= 0)
          (*qt)[static_cast<size_t>(d.qtoff) + static_cast<size_t>(k) * d.mstride + j] = v;
      }
  }
  if (eh) segs.push_back(CopySeg{pl.Eh, reinterpret_cast<uint8_t*>(eh->data()), pl.e_floats * 2});
  if (q) segs.push_back(CopySeg{pl.Q, reinterpret_cast<uint8_t*>(q->data()), pl.q_floats * 4});
  if (qt) segs.push_back(CopySeg{pl.QT, reinterpret_cast<uint8_t*>(qt->data()), pl.qt_floats * 4});
  pl.q_ready = sb.has_q;
  return POWERSGD_OK;
}

}  // namespace
}  // extern "C++"

powersgd_status powersgd_state_export(powersgd_state* st, void* host_buf, int64_t capacity,
                                      int64_t* size, void* stream) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (!size) return fail(POWERSGD_ERR_INVALID_ARG, "size is NULL");
  SnapWriter measure;
  write_snapshot(st, measure, nullptr);
  *size = measure.pos;
  if (!host_buf) return POWERSGD_OK;
  if (capacity < measure.pos)
    return fail(POWERSGD_ERR_INVALID_ARG, "capacity " + std::to_string(capacity) +
                                              " is below the snapshot's " +
                                              std::to_string(measure.pos) + " bytes");
  HipDeviceGuard guard(st->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // buckets whose E's place holds M': their error, materialized for the copies
  for (auto& kv : st->buckets) {
    BucketPlan& pl = *kv.second;
    if (pl.keeps_mprime() && (!pl.w_holds_e || pl.wstride != 0)) {
      const float* src = nullptr;
      powersgd_status r = error_source(pl, s, &src);
      if (r != POWERSGD_OK) return r;
    }
  }
  SnapWriter w;
  w.base = static_cast<uint8_t*>(host_buf);
  ExportCopies copies;
  write_snapshot(st, w, &copies);
  powersgd_status r = staged_copy(copies.segs, true, s);
  if (r != POWERSGD_OK) return r;
  for (const ExportCopies::EPiece& ep : copies.epieces) {
    const uint16_t* src = copies.ebufs[ep.ebuf].data() + ep.eoff;
    for (int64_t i = 0; i < ep.count; ++i) {
      const float v = host_from_h16(src[i], ep.prec);
      std::memcpy(ep.dst + i * 4, &v, 4);
    }
  }
  for (const ExportCopies::QPiece& qp : copies.qpieces) {
    const float* src = copies.qbufs[qp.qbuf].data() + qp.qoff;
    for (int32_t j = 0; j < qp.m; ++j)
      std::memcpy(qp.dst + static_cast<size_t>(j) * qp.rank * 4,
                  src + static_cast<size_t>(j) * qp.R, static_cast<size_t>(qp.rank) * 4);
  }
  return POWERSGD_OK;
}

powersgd_status powersgd_state_import(powersgd_state* st, const void* host_buf, int64_t size,
                                      void* stream) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  if (!host_buf || size < 0) return fail(POWERSGD_ERR_INVALID_ARG, "snapshot buffer is NULL or size < 0");
  const powersgd_hparams& hp = st->hp;
  SnapReader rd{static_cast<const uint8_t*>(host_buf), size};
  char magic[8];
  for (char& c : magic)
    if (!rd.get(c)) return snap_bad("truncated header");
  if (std::memcmp(magic, kSnapMagic, 8) != 0) return snap_bad("bad magic");
  uint32_t version = 0, flags = 0, reserved = 0;
  int32_t rank = 0;
  double rate = 0.0;
  uint64_t seed = 0;
  int64_t iteration = 0, numel_in = 0, numel_comm = 0, next_log = 0, nbuckets = 0;
  if (!rd.get(version)) return snap_bad("truncated header");
  if (version != kSnapVersion) return snap_bad("unknown version " + std::to_string(version));
  if (!rd.get(flags) || !rd.get(rank) || !rd.get(reserved) || !rd.get(rate) || !rd.get(seed) ||
      !rd.get(iteration) || !rd.get(numel_in) || !rd.get(numel_comm) || !rd.get(next_log) ||
      !rd.get(nbuckets))
    return snap_bad("truncated header");
  if (reserved != 0 || (flags & ~3u) != 0) return snap_bad("bad flags");
  if (flags != snap_flags(hp) || rank != hp.matrix_approximation_rank ||
      std::memcmp(&rate, &hp.min_compression_rate, sizeof(double)) != 0 || seed != hp.random_seed)
    return snap_bad("taken under other hyperparameters (error feedback, warm start, rank, "
                    "min_compression_rate or random_seed differ)");
  if (iteration < 0 || numel_in < 0 || numel_comm < 0 || next_log < 0 || nbuckets < 0)
    return snap_bad("negative counter");
  if (nbuckets > (rd.size - rd.pos) / 32) return snap_bad("truncated bucket records");

  std::vector<SnapBucket> parsed(static_cast<size_t>(nbuckets));
  int64_t prev = INT64_MIN;
  for (SnapBucket& sb : parsed) {
    if (prev == INT64_MAX) return snap_bad("bucket indices not strictly ascending");
    powersgd_status r = read_bucket(hp, rd, prev, sb);
    if (r != POWERSGD_OK) return r;
    prev = sb.index;
  }
  if (rd.pos != rd.size) return snap_bad(std::to_string(rd.size - rd.pos) + " trailing bytes");

  HipDeviceGuard guard(st->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::list<std::vector<float>> keep;  // stable addresses while the lists grow
  std::list<std::vector<uint16_t>> keep16;
  std::vector<CopySeg> segs;
  powersgd_status r = POWERSGD_OK;
  for (SnapBucket& sb : parsed) {
    r = upload_bucket(hp, sb, s, segs, keep, keep16);
    if (r != POWERSGD_OK) break;
  }
  if (r == POWERSGD_OK) r = staged_copy(segs, false, s);
  if (r != POWERSGD_OK) {
    (void)hipStreamSynchronize(s);  // allocation work of the new plans, before they are freed
    return r;
  }

  std::map<int64_t, std::unique_ptr<BucketPlan>> fresh;
  for (SnapBucket& sb : parsed) fresh.emplace(sb.index, std::move(sb.plan));
  st->buckets.swap(fresh);  // the old plans are released with `fresh`
  st->passthrough.clear();
  st->iteration = iteration;
  st->numel_in = numel_in;
  st->numel_comm = numel_comm;
  st->next_log_iteration = next_log;
  return POWERSGD_OK;
}

powersgd_status powersgd_set_timing(powersgd_state* st, int32_t enable) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  HipDeviceGuard guard(st->device);
  collect_timing(st);
  st->timing = enable != 0;
  for (int k = 0; k < POWERSGD_NUM_KERNELS; ++k) {
    st->t_ms[k] = 0.0;
    st->t_count[k] = 0;
    st->t_bytes[k] = 0.0;
  }
  return POWERSGD_OK;
}

powersgd_status powersgd_get_kernel_times(powersgd_state* st, double* ms, int64_t* launches,
                                          double* bytes) {
  if (!st) return fail(POWERSGD_ERR_INVALID_ARG, "state is NULL");
  HipDeviceGuard guard(st->device);
  collect_timing(st);
  for (int k = 0; k < POWERSGD_NUM_KERNELS; ++k) {
    if (ms) ms[k] = st->t_ms[k];
    if (launches) launches[k] = st->t_count[k];
    if (bytes) bytes[k] = st->t_bytes[k];
  }
  return POWERSGD_OK;
}

}  // extern "C"
