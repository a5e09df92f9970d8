// Split of ring launches over the XCDs of the GPU, sized by per-XCD speeds.
//
// The eight dies of one GPU do not run the ring kernel at the same speed (a few
// percent apart per tile), so with an equal split the slowest die ends the
// launch alone.  By default every launch splits equally and this file does
// nothing at launch time.  A caller can give the speeds (FIXED mode), or ask
// for them to be measured (MEASURING mode): then a launch records, per XCD, the
// start of its first workgroup, the end of its last one and the summed running
// time of its workgroups; the first 64 launches and then one in 8 copy those
// values back on the caller's stream into pinned host memory (set up when the
// mode is chosen), and a later call reads them once that copy has completed
// (never waiting for it).  Work over running time gives each XCD's speed, and
// their running average sizes the next launches' split.  Under either mode a
// slow XCD hands the head of its longest-first item list to faster ones, which
// run those items first; every XCD keeps its own shortest items to end its
// list.  The split is kept only if a simulation of each XCD's list schedule
// says it ends sooner than the fixed one.  Nothing here changes what any item
// computes.
#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kTileKeys = 64;            // keys per tile of the matrix-core kernel
constexpr double kItemFixed = 3.0;       // time of an item outside its tile loop, in tiles
constexpr double kItemGap = 2.4;         // a CU's idle time between two workgroups, in tiles
constexpr int kStatWords = 3 * kXcds;    // end stamps, start stamps, busy times
constexpr int kCusPerXcd = 32;           // 256 CUs in 8 XCDs
constexpr int kMinItems = 64;            // below this many items per XCD the split stays fixed
constexpr int64_t kMaxItems = 1 << 22;   // bound on the planner's host work
constexpr unsigned long long kMask40 = (1ull << 40) - 1;
constexpr long long kMinTicks = 100000;  // launches shorter than 1 ms are not measured
constexpr int kMaxDev = 64;
constexpr int kAvgN = 8;                 // measurements averaged (see consume)
constexpr unsigned kReadAll = 64;        // launches read back one by one, then one in 8

struct Shape {
  int B, Hq, Hkv, nqblk, qlen, dev0, nkblk, klen, ntq, gpl, layout, N, blk, causal, rows, per_cu;
  bool operator==(const Shape& o) const { return memcmp(this, &o, sizeof(Shape)) == 0; }
};

Shape shape_of(const AttnParams& p, bool causal, int rows, int per_cu) {
  return Shape{p.B,     p.Hq, p.Hkv,    p.nqblk, p.qlen, p.dev0,        p.nkblk, p.klen,
               p.ntq,   p.gpl, p.layout, p.N,     p.blk,  causal ? 1 : 0, rows,    per_cu};
}

// Tiles the kernel visits for query tile t of query block qi.  Positions ascend
// inside every block, so a key block is skipped, taken whole, or taken up to its
// last tile that starts at or before the query tile's last position.
double tile_count(const Shape& s, int qi, int t) {
  const int ntile = (s.klen + kTileKeys - 1) / kTileKeys;
  if (!s.causal) return (double)s.nkblk * ntile;
  const int dev = s.dev0 + qi, a0 = t * s.rows, nrows = std::min(s.rows, s.qlen - a0);
  const int qmin = layout_pos(s.layout, s.N, s.blk, dev, a0);
  const int qmax = layout_pos(s.layout, s.N, s.blk, dev, a0 + nrows - 1);
  double n = 0;
  for (int j = 0; j < s.nkblk; ++j) {
    if (layout_pos(s.layout, s.N, s.blk, j, 0) > qmax) continue;
    if (layout_pos(s.layout, s.N, s.blk, j, s.klen - 1) <= qmin) {
      n += ntile;
      continue;
    }
    int lo = 0, hi = ntile;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (layout_pos(s.layout, s.N, s.blk, j, mid * kTileKeys) <= qmax)
        lo = mid + 1;
      else
        hi = mid;
    }
    n += lo;
  }
  return n;
}

// Work of every item in tile units, indexed as the kernel numbers items: the
// item's set of query heads within their kv head's group fastest, then the
// (query block, query tile) rank of item_tile, then kv head and batch.
std::vector<float> item_work(const Shape& s) {
  const int ngrp = (s.Hq / s.Hkv) >> s.gpl;  // items per (kv head, query tile)
  const int nt = s.nqblk * s.ntq;
  std::vector<float> per((size_t)nt);
  for (int r = 0; r < nt; ++r) {
    int qi, t;
    item_tile(s.layout, s.causal != 0, s.nqblk, s.ntq, s.rows, s.blk, r, qi, t);
    per[(size_t)r] = (float)(tile_count(s, qi, t) + kItemFixed);
  }
  const int64_t W = (int64_t)s.B * s.Hkv * ngrp * nt;
  std::vector<float> wk((size_t)W);
  for (int64_t L = 0; L < W; ++L) wk[(size_t)L] = per[(size_t)((L / ngrp) % nt)];
  return wk;
}

// Finish time of a list of items taken in order by `slots` workgroup slots, each
// taking the next item as soon as it is free (with the CU's idle gap between
// two workgroups); *work receives the list's total work.
double makespan(const XcdPlan& X, const std::vector<float>& wk, int x, int slots, double* work) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> q;
  for (int i = 0; i < slots; ++i) q.push(0.0);
  double end = 0;
  *work = 0;
  for (int sl = 0; sl < X.keep[x] + X.dcnt[x]; ++sl) {
    const int64_t L = xcd_item(X, (int64_t)sl * kXcds + x);
    const double t = q.top() + wk[(size_t)L] + kItemGap;
    q.pop();
    q.push(t);
    end = std::max(end, t);
    *work += wk[(size_t)L];
  }
  return end;
}

struct Planned {
  XcdPlan xp;
  int64_t grid;
  double ms[kXcds];    // simulated finish of each XCD, in tile units
  double work[kXcds];  // work of each XCD's items, in tile units
};

void fixed_plan(XcdPlan& X, int M) {
  memset(&X, 0, sizeof X);
  X.M = M;
  for (int x = 0; x < kXcds; ++x) X.keep[x] = M;
}

// Latest finish over the XCDs, each XCD's simulated finish divided by its speed.
double finish(Planned& P, const std::vector<float>& wk, const double* f, int slots) {
  double worst = 0;
  for (int x = 0; x < kXcds; ++x) {
    P.ms[x] = makespan(P.xp, wk, x, slots, &P.work[x]);
    worst = std::max(worst, P.ms[x] / f[x]);
  }
  return worst;
}

// Every workgroup of the grid maps to a distinct item or to none, and every
// item is taken.
bool plan_valid(const XcdPlan& X, int64_t W, int64_t grid) {
  std::vector<char> seen((size_t)W, 0);
  int64_t n = 0;
  for (int64_t w = 0; w < grid; ++w) {
    const int64_t L = xcd_item(X, w);
    if (L < 0) continue;
    if (L >= W || seen[(size_t)L]) return false;
    seen[(size_t)L] = 1;
    ++n;
  }
  return n == W;
}

// The split for per-XCD shares of the work `tgt` (in tile units, gaps
// included, summing to the whole launch): an XCD above its share gives away
// the head of its list (its longest items) and keeps the tail that fits its
// share; the items given away go, in order, to the XCDs below theirs, which
// run them before their own.  An XCD that keeps its whole list and is below
// its share receives; the last such XCD takes whatever is left.  Returns
// false when nothing moves.
bool plan_for_shares(const std::vector<float>& wk, int M, const double* tgt, Planned& pl) {
  fixed_plan(pl.xp, M);
  double kept[kXcds];
  std::vector<int64_t> donated;
  for (int x = 0; x < kXcds; ++x) {
    double own = 0;
    for (int s = 0; s < M; ++s) own += wk[(size_t)x * M + s] + kItemGap;
    kept[x] = own;
    if (own <= tgt[x]) continue;
    double cum = 0;
    int j = M;  // keep items j .. M-1
    while (j > 0 && cum + 0.5 * (wk[(size_t)x * M + j - 1] + kItemGap) < tgt[x])
      cum += wk[(size_t)x * M + --j] + kItemGap;
    pl.xp.keep[x] = M - j;
    kept[x] = cum;
    for (int s = 0; s < j; ++s) donated.push_back((int64_t)x * M + s);
  }
  if (donated.empty()) return false;
  size_t pos = 0;
  int last = -1;
  for (int x = 0; x < kXcds; ++x) {
    pl.xp.dbeg[x] = (int)pos;
    const double need = tgt[x] - kept[x];
    if (pl.xp.keep[x] < M || need <= 0) continue;
    double got = 0;
    while (pos < donated.size() && got + 0.5 * (wk[(size_t)donated[pos]] + kItemGap) < need) {
      got += wk[(size_t)donated[pos++]] + kItemGap;
      ++pl.xp.dcnt[x];
    }
    last = x;
  }
  if (last < 0) return false;
  pl.xp.dcnt[last] += (int)(donated.size() - pos);  // its slice ends where the rest begins
  int64_t slots_max = 0;
  for (int x = 0; x < kXcds; ++x)
    slots_max = std::max<int64_t>(slots_max, pl.xp.keep[x] + pl.xp.dcnt[x]);
  pl.grid = slots_max * kXcds;
  return true;
}

// The split for per-XCD speeds fin (any positive scale).  The first shares
// are the whole work times each XCD's share of the speed.  Each pass then
// simulates the XCDs' list schedules and scales every share by the mean
// simulated finish over that XCD's own (an XCD that ends late gets less, one
// that ends early more).  The plan that ends soonest is kept, if it ends
// sooner than the fixed split.
Planned make_plan(const std::vector<float>& wk, int M, const float* fin, int slots) {
  constexpr int kPasses = 8;
  double f[kXcds], fs = 0;
  for (int x = 0; x < kXcds; ++x) {
    f[x] = fin[x] > 0.f ? fin[x] : 1.0;
    fs += f[x];
  }
  Planned fixed;
  fixed_plan(fixed.xp, M);
  fixed.grid = (int64_t)M * kXcds;
  const double t_fixed = finish(fixed, wk, f, slots);

  double total = 0;
  for (size_t i = 0; i < wk.size(); ++i) total += wk[i] + kItemGap;
  double tgt[kXcds];
  for (int x = 0; x < kXcds; ++x) tgt[x] = total * f[x] / fs;
  Planned best = fixed;
  double t_best = t_fixed;
  for (int pass = 0; pass < kPasses; ++pass) {
    Planned pl;
    if (!plan_for_shares(wk, M, tgt, pl)) break;
    const double t = finish(pl, wk, f, slots);
    if (t < t_best && plan_valid(pl.xp, (int64_t)M * kXcds, pl.grid)) {
      best = pl;
      t_best = t;
    }
    // (an XCD left without items keeps its share)
    double mean = 0, sum = 0;
    int busy = 0;
    for (int x = 0; x < kXcds; ++x)
      if (pl.ms[x] > 0) {
        mean += pl.ms[x] / f[x];
        ++busy;
      }
    if (busy == 0) break;
    mean /= busy;
    for (int x = 0; x < kXcds; ++x) {
      if (pl.ms[x] > 0) tgt[x] *= mean / (pl.ms[x] / f[x]);
      sum += tgt[x];
    }
    for (int x = 0; x < kXcds; ++x) tgt[x] *= total / sum;
  }
  if (t_best < t_fixed * 0.998) return best;
  return fixed;
}

// Per device: how its ring launches are split.  EQUAL (the default) uses the
// fixed XCD-major split and touches no host state; FIXED plans for speeds the
// caller set; MEASURING records stamps and reads them back to estimate speeds.
enum Mode : int { EQUAL = 0, FIXED = 1, MEASURING = 2 };

struct DevState {
  Mode mode = EQUAL;
  bool ok = false;                      // stamp buffer and read-back set up
  unsigned long long* stat = nullptr;   // this device's g_xcd_stat
  unsigned long long* host = nullptr;   // pinned copy of it
  hipEvent_t ev = nullptr;              // completes when the copy has landed
  unsigned calls = 0;                   // tag of the latest stamped launch
  bool pending = false;
  unsigned ptag = 0;
  double pwork[kXcds] = {};
  float f[kXcds] = {1, 1, 1, 1, 1, 1, 1, 1};  // speed estimate, mean 1
  int nmeas = 0;
  bool have_shape = false;
  Shape shape{};
  std::vector<float> wk;
  bool have_plan = false;
  float pf[kXcds] = {};                 // the speeds `plan` was made for
  Planned plan{};
};

std::mutex g_mu;
DevState g_dev[kMaxDev];
std::atomic<int> g_active{0};  // devices not in EQUAL mode

// Pinned host memory and an event for the read-back (once per device, with
// that device current; kept until the process ends).
bool setup(DevState& d) {
  if (d.ok) return true;
  void* sym = xcd_stat_address();
  if (sym == nullptr) return false;
  void* h = nullptr;
  if (hipHostMalloc(&h, sizeof(unsigned long long) * kStatWords, hipHostMallocDefault) !=
      hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipHostFree(h);
    return false;
  }
  d.stat = (unsigned long long*)sym;
  d.host = (unsigned long long*)h;
  d.ev = ev;
  d.ok = true;
  return true;
}

void set_mode(DevState& d, Mode m) {
  if ((d.mode == EQUAL) != (m == EQUAL)) g_active += m == EQUAL ? -1 : 1;
  d.mode = m;
}

// Reads the stamps of the pending launch if its copy has landed.
void consume(DevState& d) {
  const hipError_t q = hipEventQuery(d.ev);
  if (q == hipErrorNotReady) {
    (void)hipGetLastError();
    return;
  }
  d.pending = false;
  if (q != hipSuccess) {
    (void)hipGetLastError();
    d.ok = false;
    return;
  }
  if (d.mode != MEASURING) return;
  const unsigned long long tag = d.ptag;
  long long t0 = LLONG_MAX;
  for (int x = 0; x < kXcds; ++x) {
    if ((d.host[kXcds + x] >> 40) != tag) return;  // overlapped by another measured launch
    t0 = std::min(t0, (long long)(d.host[kXcds + x] & kMask40));
  }
  // speed = the work of the XCD's items over the time its workgroups were
  // running (the sum over its workgroups; idle CUs at the end do not count)
  double meas[kXcds], sum = 0;
  for (int x = 0; x < kXcds; ++x) {
    const long long dur = (long long)(d.host[x] & kMask40) - t0;
    const double busy = (double)d.host[2 * kXcds + x];
    if (dur < kMinTicks || !(busy > 0)) return;
    meas[x] = d.pwork[x] / busy;
    sum += meas[x];
  }
  double lo = 1e300, hi = 0;
  for (int x = 0; x < kXcds; ++x) {
    meas[x] *= kXcds / sum;
    lo = std::min(lo, meas[x]);
    hi = std::max(hi, meas[x]);
  }
  // XCDs differ by a few percent; a wider spread means a launch that was not
  // alone on the GPU, a clock ramp, or work too coarse for the model
  if (hi > 1.25 * lo) return;
  // One launch's speeds scatter by a few percent around each XCD's own level:
  // the mean of the first kAvgN measurements, then a running average that
  // gives each new one a weight of 1 / kAvgN.
  const double a = 1.0 / std::min(d.nmeas + 1, kAvgN);
  double fsum = 0, g[kXcds];
  for (int x = 0; x < kXcds; ++x) {
    g[x] = (1.0 - a) * d.f[x] + a * meas[x];
    fsum += g[x];
  }
  for (int x = 0; x < kXcds; ++x) d.f[x] = (float)(g[x] * kXcds / fsum);
  ++d.nmeas;
}

}  // namespace

int64_t xcd_prepare(const AttnParams& p, int64_t nwg, bool causal, bool ring, int rows,
                    int per_cu, hipStream_t s, XcdPlan* X) {
  memset(X, 0, sizeof *X);
  if (nwg % kXcds != 0 || nwg / kXcds > INT_MAX) return nwg;
  const int M = (int)(nwg / kXcds);
  fixed_plan(*X, M);
  // the default: every device splits equally, and nothing below runs
  if (!ring || M < kMinItems || nwg > kMaxItems || g_active.load() == 0) return nwg;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return nwg;
  }
  // The launch runs on the stream's device.  Copies and events act on the
  // current device, so a launch on another device's stream uses that device's
  // split but is not measured.
  hipDevice_t sdev = dev;
  if (s != nullptr &&
      (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev < 0 || sdev >= kMaxDev)) {
    (void)hipGetLastError();
    return nwg;
  }
  const bool here = sdev == dev;
  std::lock_guard<std::mutex> lock(g_mu);
  DevState& d = g_dev[sdev];
  if (d.mode == EQUAL) return nwg;
  bool capturing = false;
  if (d.mode == MEASURING) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    capturing = hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
    (void)hipGetLastError();
    if (!capturing && here && d.pending) consume(d);  // no event query inside a capture
  }
  const Shape sh = shape_of(p, causal, rows, per_cu);
  if (!d.have_shape || !(sh == d.shape)) {
    d.wk = item_work(sh);
    d.shape = sh;
    d.have_shape = true;
    d.have_plan = false;
  }
  // replan when a speed has moved by more than 0.2 % since the plan was made
  float moved = 0.f;
  for (int x = 0; x < kXcds; ++x) moved = std::max(moved, std::fabs(d.pf[x] - d.f[x]));
  if (!d.have_plan || moved > 0.002f) {
    d.plan = make_plan(d.wk, M, d.f, kCusPerXcd * per_cu);
    memcpy(d.pf, d.f, sizeof d.f);
    d.have_plan = true;
  }
  *X = d.plan.xp;
  if (d.mode == MEASURING && d.ok && !capturing && here) {
    d.calls = (d.calls + 1) & 0xFFFFFF;
    if (d.calls == 0) d.calls = 1;
    X->tag = (unsigned long long)d.calls << 40;
  }
  return d.plan.grid;
}

void xcd_after_launch(const XcdPlan& X, hipStream_t s) {
  if (X.tag == 0) return;  // only measured launches (MEASURING mode) carry a tag
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DevState& d = g_dev[dev];
  const unsigned tag = (unsigned)(X.tag >> 40);
  if (d.mode != MEASURING || !d.ok || d.pending || !(tag <= kReadAll || tag % 8 == 0)) return;
  if (hipMemcpyAsync(d.host, d.stat, sizeof(unsigned long long) * kStatWords,
                     hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipEventRecord(d.ev, s) != hipSuccess) {
    (void)hipGetLastError();
    d.ok = false;
    return;
  }
  d.pending = true;
  d.ptag = tag;
  memcpy(d.pwork, d.plan.work, sizeof d.pwork);
}

int64_t xcd_plan_for(const AttnParams& p, int64_t nwg, bool causal, int rows, int per_cu,
                     const float* speeds, XcdPlan* out) {
  memset(out, 0, sizeof *out);
  if (nwg % kXcds != 0 || nwg / kXcds > INT_MAX) return 0;
  const int M = (int)(nwg / kXcds);
  if (M < kMinItems || nwg > kMaxItems) return 0;
  const Planned pl =
      make_plan(item_work(shape_of(p, causal, rows, per_cu)), M, speeds, kCusPerXcd * per_cu);
  *out = pl.xp;
  return pl.grid;
}

int xcd_speeds(float* speeds, int* nmeas, int set) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return -1;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DevState& d = g_dev[dev];
  if (set == 1 || set == 2) {
    double sum = 0;
    const bool given = set == 1 && speeds != nullptr;
    for (int x = 0; x < kXcds; ++x) {
      const float v = given ? speeds[x] : 1.f;
      if (!(v > 0.f) || v > 1e6f) return -2;
      sum += v;
    }
    if (set == 2 && !setup(d)) return -3;
    for (int x = 0; x < kXcds; ++x) d.f[x] = (float)((given ? speeds[x] : 1.f) * kXcds / sum);
    d.nmeas = 0;
    d.pending = false;  // a copy in flight is dropped: its launch used other speeds
    set_mode(d, set == 2 ? MEASURING : (given ? FIXED : EQUAL));
    return 0;
  }
  if (speeds)
    for (int x = 0; x < kXcds; ++x) speeds[x] = d.f[x];
  if (nmeas) *nmeas = d.nmeas;
  return d.mode;
}

}  // namespace ra
