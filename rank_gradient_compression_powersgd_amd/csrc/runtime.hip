// C ABI of libpsgd.so: contexts, plans (validated descriptor tables + workspace) and the three
// step calls, each enqueuing grouped kernels on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "../../include/psgd.h"
#include "psgd_internal.h"

namespace psgd {
int ef_mq_rows_per_block();
int mtp_cols_per_block();
int mtp_rows_per_stage();
int gs_apply_rows_per_block();
int decomp_tile_m();
int decomp_tile_n();
}  // namespace psgd

using psgd::DevMat;
using psgd::Work;

struct psgd_plan;

struct psgd_ctx {
  int device = 0;
  int rank = 0;
  std::string err;
  std::vector<hipEvent_t> events;   // tracing hook: 2 per slot, empty when off
  char* scratch = nullptr;          // device address of this device's static scratch array
  std::unique_ptr<psgd_plan> noalloc_plan;   // host side of psgd_step_noalloc's transient plan
};

// ------------------------------------------------------------------------------------------
// Static device scratch for psgd_step_noalloc: the workspace, descriptor table and work lists
// of one group live here, so that entry point allocates nothing. Each device holds its own
// copy of the array, from the first context created on it until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a stand-in): the device
// address comes from hipGetSymbolAddress, taken once per device in psgd_create with that
// device current, and kept in g_scratch_addr.
// ------------------------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;      // 32 MiB per device
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices] = {nullptr};
}  // namespace
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

enum WorkKind { W_K1, W_GRAM, W_REDUCE, W_FACTOR, W_BGEMM, W_APPLY, W_K2, W_SPLIT3, W_SPLITQ, W_K3,
                W_SPLITM, W_SPLITQT, W_G1, W_G2, W_KINDS };
constexpr int kMaxBlocks = psgd::kMaxRank / psgd::kBlk;   // 128-column blocks of the largest rank

}  // namespace

struct psgd_plan {
  psgd_ctx* ctx = nullptr;
  size_t praw_bytes = 0;   // the contiguous raw-factor region at the start of the workspace
  int n_mats = 0, n_blocks = 0, gt = 0, rt = 0, rtc = 0, chunks = 0;
  bool big = false;   // rank above one 128-column block: blocked orthonormalisation
  std::vector<DevMat> mats;
  DevMat* d_mats = nullptr;
  void* workspace = nullptr;
  size_t ws_bytes = 0;
  Work* d_work = nullptr;
  int off[W_KINDS] = {0};
  int cnt[W_KINDS] = {0};
  int nblk = 1;                          // 128-column blocks of rpad
  int bg_off[kMaxBlocks][2] = {{0}};     // block products of step k, phase 0/1 (within W_BGEMM)
  int bg_cnt[kMaxBlocks][2] = {{0}};
  int32_t* d_one = nullptr;              // a device word holding 1: the decompression's skip
                                         // word for psgd_reset_errors
  int64_t* d_counters = nullptr;         // steps decompressed, steps skipped
  // optimizer attachment (psgd_adam_attach)
  int adam_pt = 0;                       // parameter type, 0 = none attached
  void* adam_buf = nullptr;              // norm items (q_next ranges, then pass-through ranges)
                                         // and their fp64 sums
  psgd::NormItem* d_items = nullptr;
  double* d_partial = nullptr;
  int n_plan_items = 0;
};

namespace {

psgd_status fail(psgd_ctx* ctx, psgd_status st, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
psgd_status fail(psgd_ctx* ctx, psgd_status st, const char* fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->err = buf;
  }
  return st;
}

psgd_status hip_fail(psgd_ctx* ctx, hipError_t e, const char* what) {
  return fail(ctx, PSGD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

enum Slot { S_ZERO_FLAGS, S_K1, S_GRAM, S_FACTOR, S_APPLY, S_K2, S_ZERO_SKIP, S_CHECK,
            S_K3, S_REDUCE, S_SPLIT3, S_REORTH, S_ADAM_NORM, S_K3_ADAM, S_ADAM_PASS, S_SLOTS };
constexpr int kMaxPassItems = 8192;      // norm items of pass-through gradients per call

// Launch `expr` in tracing slot `slot`, bracketed by the hook's events when installed.
template <typename F>
hipError_t traced(psgd_ctx* ctx, int slot, hipStream_t s, F&& launch) {
  if (!ctx->events.empty()) {
    const hipError_t e = hipEventRecord(ctx->events[2 * slot], s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch();
  if (e != hipSuccess || ctx->events.empty()) return e;
  return hipEventRecord(ctx->events[2 * slot + 1], s);
}

#define HIPCHK(ctx, expr, what)                         \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, what); \
  } while (0)

inline int64_t rup(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

int psgd_version(void) { return PSGD_ABI_VERSION; }

psgd_status psgd_create(psgd_ctx** out, int device, int rank) {
  if (!out) return PSGD_EINVAL;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return PSGD_EINVAL;
  if (rank < 1) return PSGD_EINVAL;
  if (rank > psgd::kMaxRank) return PSGD_EUNSUPPORTED;
  if (device >= kMaxDevices) return PSGD_EUNSUPPORTED;
  char* scratch_addr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[device]) {
      int prev = 0;
      if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) return PSGD_EHIP;
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      (void)hipSetDevice(prev);
      if (e != hipSuccess || !ptr) return PSGD_EHIP;
      g_scratch_addr[device] = static_cast<char*>(ptr);
    }
    scratch_addr = g_scratch_addr[device];
  }
  psgd_ctx* c = new (std::nothrow) psgd_ctx;
  if (!c) return PSGD_ENOMEM;
  c->device = device;
  c->rank = rank;
  c->scratch = scratch_addr;
  c->noalloc_plan.reset(new (std::nothrow) psgd_plan);
  if (!c->noalloc_plan) {
    delete c;
    return PSGD_ENOMEM;
  }
  *out = c;
  return PSGD_OK;
}

psgd_status psgd_destroy(psgd_ctx* ctx) {
  delete ctx;
  return PSGD_OK;
}

const char* psgd_last_error(const psgd_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

}  // extern "C"

namespace {

// Workspace offsets of one matrix's buffers (bytes from the workspace base).
struct PlanOff {
  size_t p_raw, pth, ptl, p3e, q3e, p3h, q3h, gram, tmat, wsum, wdiag, p2, reorth, mh, ml, qth, qtl;
};
struct PlanLayout {
  std::vector<PlanOff> offs;
  std::vector<Work> all;       // every work list, concatenated (offsets in psgd_plan::off)
  size_t ws = 0;               // workspace bytes (a multiple of 256)
  size_t one_off = 0;          // offset of the constant word 1
  size_t counters_off = 0;     // offset of the two step counters
  size_t praw_total = 0;       // bytes of the contiguous raw-factor region at offset 0
};

// Validate a group and lay out its plan on the host: descriptors (workspace pointers still
// unbound), grouped work lists and the workspace offsets. Shared by psgd_plan_create, which
// allocates the workspace, and psgd_step_noalloc, which places it in the library's static
// scratch array.
psgd_status plan_layout(psgd_ctx* ctx, const psgd_matrix* mats, int n_mats, psgd_dtype grad_dtype,
                        int n_blocks, psgd_plan* p, PlanLayout& L) {
  if (!mats || n_mats < 1) return fail(ctx, PSGD_EINVAL, "need at least one matrix");
  if (n_blocks < 1) return fail(ctx, PSGD_EINVAL, "n_blocks must be >= 1");
  int gt = 0;
  switch (grad_dtype) {
    case PSGD_F16: gt = psgd::G_F16; break;
    case PSGD_BF16: gt = psgd::G_BF16; break;
    case PSGD_F32: gt = psgd::G_F32; break;
    default: return fail(ctx, PSGD_EDTYPE, "unknown gradient dtype %d", (int)grad_dtype);
  }
  // Rank layout. The streaming product kernels carry at most kMaxRankTiles 16-column tiles, so
  // ranks above 128 (which take the split-once GEMM path instead) are laid out as `chunks`
  // equal chunks of `rtc` tiles; rpad = chunks * rtc * 16 >= r, the extra factor columns stay
  // zero. The 128-column blocks of the orthonormalisation follow the same padding.
  const int r = ctx->rank;
  const int rt0 = (int)(rup(r, 16) / 16);
  const int chunks = (rt0 + psgd::kMaxRankTiles - 1) / psgd::kMaxRankTiles;
  const int rtc = (rt0 + chunks - 1) / chunks;
  const int rt = chunks * rtc;
  const int rpad = rt * 16;
  const int kpad3 = (int)rup(r, 32);
  const bool big = rpad > psgd::kBlk;
  p->ctx = ctx;
  p->n_mats = n_mats;
  p->n_blocks = n_blocks;
  p->gt = gt;
  p->rt = rt;
  p->rtc = rtc;
  p->chunks = chunks;
  p->big = big;

  // ---- validate and lay out the workspace ---------------------------------------------
  // The raw factors M q of all matrices come first, as one contiguous region (the buffer a
  // data-parallel caller all-reduces between psgd_compress_p and psgd_orthogonalize).
  size_t praw_total = 0;
  for (int i = 0; i < n_mats; ++i)
    if (mats[i].m >= 1 && mats[i].m <= (1 << 28)) praw_total += (size_t)mats[i].m * rpad * 4;
  size_t praw_cursor = 0;
  size_t ws = (size_t)rup((int64_t)praw_total, 256);
  auto take = [&](size_t bytes) { size_t o = ws; ws += (size_t)rup((int64_t)bytes, 256); return o; };
  std::vector<PlanOff>& offs = L.offs;
  offs.assign(n_mats, PlanOff{});
  p->mats.resize(n_mats);
  for (int i = 0; i < n_mats; ++i) {
    const psgd_matrix& a = mats[i];
    if (!a.err || !a.q || !a.q_next || !a.p)
      return fail(ctx, PSGD_EINVAL, "matrix %d: err, q, q_next and p are required", i);
    if (a.m < 1 || a.n < 1 || a.m > (1 << 28) || a.n > (1 << 28))
      return fail(ctx, PSGD_EINVAL, "matrix %d: bad shape %lld x %lld", i, (long long)a.m, (long long)a.n);
    if (a.n % 8 != 0) return fail(ctx, PSGD_EINVAL, "matrix %d: n = %lld is not a multiple of 8", i, (long long)a.n);
    if (r > a.m || r > a.n)
      return fail(ctx, PSGD_EINVAL, "matrix %d: rank %d exceeds min(m, n)", i, r);
    if (a.grad && (a.ld_grad < a.n || a.ld_grad % 8 != 0))
      return fail(ctx, PSGD_EINVAL, "matrix %d: ld_grad must be >= n and a multiple of 8", i);
    if (a.ld_err < a.n || a.ld_err % 4 != 0)
      return fail(ctx, PSGD_EINVAL, "matrix %d: ld_err must be >= n and a multiple of 4", i);
    if (a.out && (a.ld_out < a.n || a.ld_out % 4 != 0))
      return fail(ctx, PSGD_EINVAL, "matrix %d: ld_out must be >= n and a multiple of 4", i);
    if (!aligned16(a.grad) || !aligned16(a.err) || !aligned16(a.q) || !aligned16(a.q_next) ||
        !aligned16(a.p) || (a.out && !aligned16(a.out)))
      return fail(ctx, PSGD_EINVAL, "matrix %d: every pointer must be 16-byte aligned", i);
    if (a.block < 0 || a.block >= n_blocks)
      return fail(ctx, PSGD_EINVAL, "matrix %d: block %d outside [0, %d)", i, a.block, n_blocks);
    if (a.reserved != 0) return fail(ctx, PSGD_EINVAL, "matrix %d: reserved field must be 0", i);

    DevMat& d = p->mats[i];
    std::memset(&d, 0, sizeof d);
    d.grad = a.grad; d.ld_grad = a.ld_grad;
    d.err = a.err; d.ld_err = a.ld_err;
    d.q = a.q; d.q_next = a.q_next; d.p = a.p;
    d.out = a.out; d.ld_out = a.ld_out;
    d.m = (int)a.m; d.n = (int)a.n; d.block = a.block; d.r = r;
    d.rpad = rpad; d.kpad3 = kpad3;
    // P^T covers whole M^T P stages and, for ranks above 128, whole split tiles (powers of two)
    d.mpad = (int)rup(a.m, std::max(psgd::mtp_rows_per_stage(), psgd::big_split_tile()));
    d.gram_rows = big ? psgd::kGramRowsBig : psgd::kGramRows;
    d.gram_parts = (int)((a.m + d.gram_rows - 1) / d.gram_rows);
    const int gsz = gt == psgd::G_F32 ? 4 : 2;
    const int64_t gb = a.grad ? ((a.m - 1) * a.ld_grad + a.n) * gsz : 0;   // no G: every load reads 0
    const int64_t eb = ((a.m - 1) * a.ld_err + a.n) * 4;
    const int64_t ob = a.out ? ((a.m - 1) * a.ld_out + a.n) * 4 : 0;
    if (gb >= (int64_t(1) << 31) || eb >= (int64_t(1) << 31) || ob >= (int64_t(1) << 31) ||
        a.n * r * 4 >= (int64_t(1) << 31) || a.m * r * 4 >= (int64_t(1) << 31))
      return fail(ctx, PSGD_EINVAL, "matrix %d: G, E, out, q and p must each span less than 2 GiB", i);
    d.g_bytes = (uint32_t)gb;
    d.e_bytes = (uint32_t)eb;
    d.o_bytes = (uint32_t)ob;
    PlanOff& o = offs[i];
    o.p_raw = praw_cursor;
    praw_cursor += (size_t)a.m * rpad * 4;
    o.pth = take((size_t)rpad * d.mpad * 2);
    o.ptl = take((size_t)rpad * d.mpad * 2);
    const int64_t m3 = rup(a.m, psgd::decomp_tile_m()), n3 = rup(a.n, psgd::decomp_tile_n());
    o.p3e = take((size_t)m3 * 4);              // zero rows up to a whole decompression tile
    o.q3e = take((size_t)n3 * 4);
    if (big) {
      // the decompression's factors split once per step (fp16 hi + lo, 4 bytes per entry)
      if (m3 * kpad3 * 4 >= (int64_t(1) << 31) || n3 * kpad3 * 4 >= (int64_t(1) << 31))
        return fail(ctx, PSGD_EINVAL, "matrix %d: the split decompression factors must each span less than 2 GiB", i);
      o.p3h = take((size_t)m3 * kpad3 * 4);
      o.q3h = take((size_t)n3 * kpad3 * 4);
    }
    o.gram = take((size_t)d.gram_parts * rpad * rpad * 8);
    o.tmat = take((size_t)rpad * rpad * 8);
    o.wsum = big ? take((size_t)rpad * rpad * 8) : 0;
    o.wdiag = big ? take((size_t)rpad * 8) : 0;
    o.p2 = take((size_t)a.m * rpad * 4);
    o.reorth = take(4);
    d.npad_b = (int)rup(a.n, psgd::big_split_tile());
    d.rpad_b = (int)rup(rpad, psgd::big_gemm_tile_n());
    if (big) {
      // the split operands of the two factor GEMMs: M (4 bytes per element of the padded
      // matrix; M^T P reads it K-outer) and q^T; each half addressed through a buffer range
      // below 2 GiB
      const size_t mb = (size_t)d.mpad * d.npad_b * 2, qb = (size_t)d.rpad_b * d.npad_b * 2;
      if (mb >= (size_t(1) << 31))
        return fail(ctx, PSGD_EINVAL, "matrix %d: %d x %d is too large for ranks above 128 (each bf16 half of M must span less than 2 GiB)", i, (int)a.m, (int)a.n);
      o.mh = take(mb); o.ml = take(mb);
      o.qth = take(qb); o.qtl = take(qb);
    }
  }

  L.one_off = take(4);
  L.counters_off = take(16);

  // ---- work lists -------------------------------------------------------------------------
  std::vector<Work>& all = L.all;
  all.clear();
  std::vector<int64_t> cost;   // bytes one item streams (same index as `all`)
  auto begin_kind = [&](int k) { p->off[k] = (int)all.size(); };
  // Padded lists are launched with xcd_remap: XCD x walks the x-th eighth of the list in order.
  // For the two long-running product kernels, whose items differ in length (2.7x within the
  // sharded resblock, 4x across the unsharded one), the list is cut into eight contiguous
  // ranges of about equal total cost rather than equal item count (each range then padded
  // with empty items to the longest), and each range is sorted by decreasing cost (stable, so
  // the blocks of one matrix stay together and share its factor in that XCD's L2): every XCD
  // gets the same work, its longest items start first and the short ones fill the tail
  // (longest-processing-time-first list scheduling).
  auto end_kind = [&](int k, bool pad8, bool sort = false) {
    cost.resize(all.size(), 0);
    if (sort) {
      const int beg = p->off[k], n = (int)all.size() - beg;
      int64_t total = 0;
      for (int j = 0; j < n; ++j) total += cost[beg + j];
      int cut[psgd::kXcds + 1];
      cut[0] = 0;
      int64_t run = 0;
      for (int x = 1, j = 0; x <= psgd::kXcds; ++x) {
        const int64_t goal = x == psgd::kXcds ? INT64_MAX : (total * x + psgd::kXcds / 2) / psgd::kXcds;
        while (j < n && run + cost[beg + j] / 2 < goal) run += cost[beg + j++];
        cut[x] = x == psgd::kXcds ? n : j;
      }
      int per = 0;
      for (int x = 0; x < psgd::kXcds; ++x) per = std::max(per, cut[x + 1] - cut[x]);
      std::vector<Work> out;
      std::vector<int64_t> oc;
      for (int x = 0; x < psgd::kXcds; ++x) {
        std::vector<int> idx;
        for (int j = cut[x]; j < cut[x + 1]; ++j) idx.push_back(beg + j);
        std::stable_sort(idx.begin(), idx.end(), [&](int u, int v) { return cost[u] > cost[v]; });
        for (int u : idx) { out.push_back(all[u]); oc.push_back(cost[u]); }
        for (int j = (int)idx.size(); j < per; ++j) { out.push_back(Work{-1, 0, 0, 0}); oc.push_back(0); }
      }
      all.resize(beg);
      cost.resize(beg);
      all.insert(all.end(), out.begin(), out.end());
      cost.insert(cost.end(), oc.begin(), oc.end());
    } else if (pad8) {
      while ((all.size() - p->off[k]) % psgd::kXcds) all.push_back(Work{-1, 0, 0, 0});
      cost.resize(all.size(), 0);
    }
    p->cnt[k] = (int)all.size() - p->off[k];
  };
  // GEMM lists: the rank tiles of one row tile form a group that shares its A tile in one XCD's
  // L2. Groups go to the XCD with the least work so far, longest first, so that each XCD gets
  // its share of the long items (contiguous eighths of the matrix-ordered list gave the XCDs
  // holding the 15872-long products up to twice the others' work at r = 896); each XCD's
  // segment, longest first, is then padded to the longest segment.
  auto end_kind_groups = [&](int k, int gsize) {
    cost.resize(all.size(), 0);
    const int beg = p->off[k], n = (int)all.size() - beg;
    std::vector<int> gstart;
    for (int j = 0; j < n; j += gsize) gstart.push_back(j);
    auto gcost = [&](int gi) {
      int64_t c = 0;
      for (int j = gstart[gi]; j < std::min(n, gstart[gi] + gsize); ++j) c += cost[beg + j];
      return c;
    };
    std::vector<int> order(gstart.size());
    for (size_t gi = 0; gi < order.size(); ++gi) order[gi] = (int)gi;
    std::stable_sort(order.begin(), order.end(), [&](int u, int v) { return gcost(u) > gcost(v); });
    std::vector<std::vector<int>> seg(psgd::kXcds);
    int64_t load[psgd::kXcds] = {};
    for (int gi : order) {
      int x = 0;
      for (int y = 1; y < psgd::kXcds; ++y) if (load[y] < load[x]) x = y;
      load[x] += gcost(gi);
      for (int j = gstart[gi]; j < std::min(n, gstart[gi] + gsize); ++j) seg[x].push_back(beg + j);
    }
    size_t per = 0;
    for (const auto& sg : seg) per = std::max(per, sg.size());
    std::vector<Work> out;
    std::vector<int64_t> oc;
    for (const auto& sg : seg) {
      for (int u : sg) { out.push_back(all[u]); oc.push_back(cost[u]); }
      for (size_t j = sg.size(); j < per; ++j) { out.push_back(Work{-1, 0, 0, 0}); oc.push_back(0); }
    }
    all.resize(beg);
    cost.resize(beg);
    all.insert(all.end(), out.begin(), out.end());
    cost.insert(cost.end(), oc.begin(), oc.end());
    p->cnt[k] = (int)all.size() - p->off[k];
  };
  auto push = [&](Work w, int64_t c) {
    all.push_back(w);
    cost.resize(all.size(), 0);
    cost.back() = c;
  };
  const int k1rows = psgd::ef_mq_rows_per_block();
  const int k2cols = psgd::mtp_cols_per_block();
  const int aprows = psgd::gs_apply_rows_per_block();
  const int tm = psgd::decomp_tile_m(), tn = psgd::decomp_tile_n();
  // streaming products (r <= 128: a single rank chunk)
  begin_kind(W_K1);
  if (!big)
    for (int i = 0; i < n_mats; ++i)
      for (int r0 = 0; r0 < p->mats[i].m; r0 += k1rows)
        for (int ch = 0; ch < p->chunks; ++ch)
          push(Work{i, r0, ch, 0}, (int64_t)std::min(k1rows, p->mats[i].m - r0) * p->mats[i].n);
  end_kind(W_K1, true, true);
  // r > 128: split tiles of M (the padded range) and of q, then the two GEMMs' C tiles (rank
  // tiles of one row tile adjacent, so they share the A tile in their XCD's L2)
  const int stile = psgd::big_split_tile(), gtm = psgd::big_gemm_tile_m(), gtn = psgd::big_gemm_tile_n();
  begin_kind(W_SPLITM);
  if (big)
    for (int i = 0; i < n_mats; ++i)
      for (int i0 = 0; i0 < p->mats[i].mpad; i0 += stile)
        for (int j0 = 0; j0 < p->mats[i].npad_b; j0 += stile) push(Work{i, i0, j0, 0}, 1);
  end_kind(W_SPLITM, true);
  begin_kind(W_SPLITQT);
  if (big)
    for (int i = 0; i < n_mats; ++i)
      for (int i0 = 0; i0 < p->mats[i].npad_b; i0 += stile)
        for (int j0 = 0; j0 < p->mats[i].rpad_b; j0 += stile) push(Work{i, i0, j0, 0}, 1);
  end_kind(W_SPLITQT, true);
  begin_kind(W_G1);
  if (big)
    for (int i = 0; i < n_mats; ++i)
      for (int i0 = 0; i0 < p->mats[i].m; i0 += gtm)
        for (int j0 = 0; j0 < rpad; j0 += gtn) push(Work{i, i0, j0, 0}, (int64_t)p->mats[i].n);
  end_kind_groups(W_G1, (rpad + gtn - 1) / gtn);
  begin_kind(W_G2);
  if (big)
    for (int i = 0; i < n_mats; ++i)
      for (int i0 = 0; i0 < p->mats[i].n; i0 += gtm)
        for (int j0 = 0; j0 < rpad; j0 += gtn) push(Work{i, i0, j0, 1}, (int64_t)p->mats[i].mpad);
  end_kind_groups(W_G2, (rpad + gtn - 1) / gtn);
  begin_kind(W_GRAM);
  const int nblk = (rpad + psgd::kBlk - 1) / psgd::kBlk;
  for (int i = 0; i < n_mats; ++i) {
    const int gr = p->mats[i].gram_rows;
    for (int pt = 0; pt < p->mats[i].gram_parts; ++pt)
      for (int bi = 0; bi < (big ? nblk : 1); ++bi)
        for (int bj = bi; bj < (big ? nblk : 1); ++bj)
          for (int q = 0; q < (big ? 4 : 1); ++q)     // 64 x 64 quadrants (qi = q & 1, qj = q >> 1)
            push(Work{i, pt * gr, pt, bi | (bj << 8) | (q << 16)}, std::min(gr, p->mats[i].m - pt * gr));
  }
  end_kind(W_GRAM, true);
  begin_kind(W_REDUCE);
  if (big)
    for (int i = 0; i < n_mats; ++i)
      for (int64_t e0 = 0; e0 * 4096 < (int64_t)rpad * rpad; ++e0) all.push_back(Work{i, (int)e0, 0, 0});
  end_kind(W_REDUCE, false);
  begin_kind(W_FACTOR);
  for (int i = 0; i < n_mats; ++i) all.push_back(Work{i, 0, 0, 0});
  end_kind(W_FACTOR, false);
  // block products of the large-rank factorisation, grouped by step k and phase
  begin_kind(W_BGEMM);
  p->nblk = nblk;
  if (big)
    for (int kb = 0; kb < nblk; ++kb)
      for (int ph = 0; ph < 2; ++ph) {
        p->bg_off[kb][ph] = (int)all.size() - p->off[W_BGEMM];
        for (int i = 0; i < n_mats; ++i) {
          if (ph == 0) {
            for (int ib = 0; ib < kb; ++ib) all.push_back(Work{i, ib, kb, 0});        // T_ik
            for (int jb = kb + 1; jb < nblk; ++jb) all.push_back(Work{i, kb, jb, 0}); // R_kj
          } else {   // four quadrant items per block (c = qi | qj << 1)
            for (int ib = 0; ib <= kb; ++ib)
              for (int jb = kb + 1; jb < nblk; ++jb)
                for (int q = 0; q < 4; ++q) all.push_back(Work{i, ib, jb, q});   // U_ij
            for (int ib = kb + 1; ib < nblk; ++ib)
              for (int jb = ib; jb < nblk; ++jb)
                for (int q = 0; q < 4; ++q) all.push_back(Work{i, ib, jb, q});   // W_ij
          }
        }
        p->bg_cnt[kb][ph] = (int)all.size() - p->off[W_BGEMM] - p->bg_off[kb][ph];
      }
  end_kind(W_BGEMM, false);
  begin_kind(W_APPLY);
  for (int i = 0; i < n_mats; ++i)
    for (int r0 = 0; r0 < p->mats[i].m; r0 += aprows)
      for (int cb = 0; cb < (big ? nblk : 1); ++cb)   // output block cb streams cb + 1 blocks of P
        push(Work{i, r0, cb, 0}, (int64_t)std::min(aprows, p->mats[i].m - r0) * (cb + 1));
  end_kind(W_APPLY, true, big);
  begin_kind(W_K2);
  if (!big)
    for (int i = 0; i < n_mats; ++i)
      for (int c0 = 0; c0 < p->mats[i].n; c0 += k2cols)
        for (int ch = 0; ch < p->chunks; ++ch)
          push(Work{i, c0, ch, 0}, (int64_t)std::min(k2cols, p->mats[i].n - c0) * p->mats[i].m);
  end_kind(W_K2, true, true);
  begin_kind(W_SPLIT3);
  if (big)
    for (int i = 0; i < n_mats; ++i) {
      for (int r0 = 0; r0 < p->mats[i].m; r0 += 64) all.push_back(Work{i, r0, 0, 0});
      for (int r0 = 0; r0 < p->mats[i].n; r0 += 64) all.push_back(Work{i, r0, 1, 0});
    }
  end_kind(W_SPLIT3, false);
  begin_kind(W_SPLITQ);
  for (int i = 0; i < n_mats; ++i)
    for (int r0 = 0; r0 < p->mats[i].n; r0 += 64) all.push_back(Work{i, r0, 1, 0});
  end_kind(W_SPLITQ, false);
  begin_kind(W_K3);
  for (int i = 0; i < n_mats; ++i)
    for (int m0 = 0; m0 < p->mats[i].m; m0 += tm)
      for (int n0 = 0; n0 < p->mats[i].n; n0 += tn)
        push(Work{i, m0, n0, 0}, (int64_t)std::min(tm, p->mats[i].m - m0) * std::min(tn, p->mats[i].n - n0));
  end_kind(W_K3, true);
  for (int k = 0; k < W_KINDS; ++k)
    if (p->cnt[k] > 0x7fffffff / 2) return fail(ctx, PSGD_EINVAL, "work list too long");
  L.ws = ws;
  L.praw_total = praw_total;
  return PSGD_OK;
}

// Point the descriptors at a workspace whose base is `base` (device memory).
void plan_bind(psgd_plan* p, char* base, const PlanLayout& L) {
  const bool big = p->big;
  for (int i = 0; i < p->n_mats; ++i) {
    DevMat& d = p->mats[i];
    const PlanOff& o = L.offs[i];
    d.p_raw = reinterpret_cast<float*>(base + o.p_raw);
    d.pt_hi = reinterpret_cast<uint16_t*>(base + o.pth);
    d.pt_lo = reinterpret_cast<uint16_t*>(base + o.ptl);
    d.p3_exp = reinterpret_cast<int32_t*>(base + o.p3e);
    d.q3_exp = reinterpret_cast<int32_t*>(base + o.q3e);
    d.p3h = big ? reinterpret_cast<uint16_t*>(base + o.p3h) : nullptr;
    d.q3h = big ? reinterpret_cast<uint16_t*>(base + o.q3h) : nullptr;
    d.gram = reinterpret_cast<double*>(base + o.gram);
    d.tmat = reinterpret_cast<double*>(base + o.tmat);
    d.wsum = big ? reinterpret_cast<double*>(base + o.wsum) : nullptr;
    d.wdiag = big ? reinterpret_cast<double*>(base + o.wdiag) : nullptr;
    d.p2 = reinterpret_cast<float*>(base + o.p2);
    d.reorth = reinterpret_cast<int32_t*>(base + o.reorth);
    if (big) {
      d.mh = reinterpret_cast<uint16_t*>(base + o.mh);
      d.ml = reinterpret_cast<uint16_t*>(base + o.ml);
      d.qth = reinterpret_cast<uint16_t*>(base + o.qth);
      d.qtl = reinterpret_cast<uint16_t*>(base + o.qtl);
    }
  }
  p->workspace = base;
  p->ws_bytes = L.ws;
  p->praw_bytes = L.praw_total;
  p->d_one = reinterpret_cast<int32_t*>(base + L.one_off);
  p->d_counters = reinterpret_cast<int64_t*>(base + L.counters_off);
}

}  // namespace

extern "C" {

psgd_status psgd_plan_create(psgd_ctx* ctx, const psgd_matrix* mats, int n_mats,
                             psgd_dtype grad_dtype, int n_blocks, psgd_plan** plan_out) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!plan_out) return fail(ctx, PSGD_EINVAL, "plan pointer is NULL");
  *plan_out = nullptr;
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  std::unique_ptr<psgd_plan> p(new (std::nothrow) psgd_plan);
  if (!p) return fail(ctx, PSGD_ENOMEM, "out of host memory");
  PlanLayout L;
  if (psgd_status st = plan_layout(ctx, mats, n_mats, grad_dtype, n_blocks, p.get(), L); st != PSGD_OK)
    return st;
  const size_t ws = L.ws;
  const std::vector<Work>& all = L.all;

  // ---- device allocations -----------------------------------------------------------------
  void* wsp = nullptr;
  hipError_t e = hipMalloc(&wsp, ws ? ws : 256);
  if (e != hipSuccess) return fail(ctx, PSGD_ENOMEM, "workspace of %zu bytes: %s", ws, hipGetErrorString(e));
  plan_bind(p.get(), static_cast<char*>(wsp), L);
  auto cleanup = [&]() {
    if (p->workspace) (void)hipFree(p->workspace);
    if (p->d_mats) (void)hipFree(p->d_mats);
    if (p->d_work) (void)hipFree(p->d_work);
    p->workspace = nullptr;
    p->d_mats = nullptr;
    p->d_work = nullptr;
  };
  if ((e = hipMemset(p->workspace, 0, ws ? ws : 256)) != hipSuccess) { cleanup(); return hip_fail(ctx, e, "workspace clear"); }
  const int32_t one = 1;
  if ((e = hipMemcpy(p->d_one, &one, sizeof one, hipMemcpyHostToDevice)) != hipSuccess) { cleanup(); return hip_fail(ctx, e, "constant upload"); }
  if ((e = hipMalloc(&p->d_mats, sizeof(DevMat) * n_mats)) != hipSuccess) { cleanup(); return fail(ctx, PSGD_ENOMEM, "descriptor table"); }
  if ((e = hipMemcpy(p->d_mats, p->mats.data(), sizeof(DevMat) * n_mats, hipMemcpyHostToDevice)) != hipSuccess) { cleanup(); return hip_fail(ctx, e, "descriptor upload"); }
  if ((e = hipMalloc(&p->d_work, sizeof(Work) * all.size())) != hipSuccess) { cleanup(); return fail(ctx, PSGD_ENOMEM, "work lists"); }
  if ((e = hipMemcpy(p->d_work, all.data(), sizeof(Work) * all.size(), hipMemcpyHostToDevice)) != hipSuccess) { cleanup(); return hip_fail(ctx, e, "work list upload"); }
  if ((e = hipDeviceSynchronize()) != hipSuccess) { cleanup(); return hip_fail(ctx, e, "plan upload"); }
  *plan_out = p.release();
  return PSGD_OK;
}

psgd_status psgd_plan_destroy(psgd_plan* plan) {
  if (!plan) return PSGD_OK;
  (void)hipSetDevice(plan->ctx->device);
  (void)hipDeviceSynchronize();
  if (plan->workspace) (void)hipFree(plan->workspace);
  if (plan->d_mats) (void)hipFree(plan->d_mats);
  if (plan->d_work) (void)hipFree(plan->d_work);
  if (plan->adam_buf) (void)hipFree(plan->adam_buf);
  delete plan;
  return PSGD_OK;
}

namespace {
psgd_status check_call(psgd_ctx* ctx, psgd_plan* plan) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!plan || plan->ctx != ctx) return fail(ctx, PSGD_EINVAL, "plan does not belong to this context");
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  return PSGD_OK;
}
}  // namespace

psgd_status psgd_compress_p(psgd_ctx* ctx, psgd_plan* plan, const float* scale, uint8_t* flags,
                            hipStream_t stream) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  if (!scale || !flags) return fail(ctx, PSGD_EINVAL, "scale and flags are required");
  const DevMat* dm = plan->d_mats;
  auto W = [&](int k) { return plan->d_work + plan->off[k]; };
  HIPCHK(ctx, traced(ctx, S_ZERO_FLAGS, stream, [&] { return psgd::launch_zero_u8(flags, plan->n_mats, stream); }), "flag clear");
  if (plan->big) {
    HIPCHK(ctx, traced(ctx, S_K1, stream, [&] {
      hipError_t e = psgd::launch_split_m(plan->gt, dm, W(W_SPLITM), plan->cnt[W_SPLITM], scale, flags, stream);
      if (e == hipSuccess) e = psgd::launch_split_qt(dm, W(W_SPLITQT), plan->cnt[W_SPLITQT], stream);
      if (e == hipSuccess) e = psgd::launch_gemm_nt(dm, W(W_G1), plan->cnt[W_G1], false, stream);
      return e; }), "M Q");
    return PSGD_OK;
  }
  HIPCHK(ctx, traced(ctx, S_K1, stream, [&] { return psgd::launch_ef_mq(plan->gt, plan->rtc, dm, W(W_K1), plan->cnt[W_K1], scale, flags, stream); }), "M Q");
  return PSGD_OK;
}

namespace {
// One orthonormalisation pass: Gram partials, T, P_hat = P T. Large ranks sum the partials and
// factor W by 128-column blocks (diagonal block, then the block products of that step).
hipError_t orth_pass(psgd_plan* plan, int pass, hipStream_t stream, psgd_ctx* ctx, bool trace) {
  const DevMat* dm = plan->d_mats;
  auto W = [&](int k) { return plan->d_work + plan->off[k]; };
  const bool big = plan->big;
  auto run = [&](int slot, auto&& f) { return trace ? traced(ctx, slot, stream, f) : f(); };
  hipError_t e = run(S_GRAM, [&] { return psgd::launch_gs_gram(plan->rt, big, pass, dm, W(W_GRAM), plan->cnt[W_GRAM], stream); });
  if (e != hipSuccess) return e;
  if (big) {
    e = run(S_REDUCE, [&] { return psgd::launch_gs_reduce(pass, dm, W(W_REDUCE), plan->cnt[W_REDUCE], stream); });
    if (e != hipSuccess) return e;
    e = run(S_FACTOR, [&] {
      hipError_t r = hipSuccess;
      for (int kb = 0; kb < plan->nblk && r == hipSuccess; ++kb) {
        r = psgd::launch_gs_fdiag(pass, kb, dm, W(W_FACTOR), plan->cnt[W_FACTOR], stream);
        for (int ph = 0; ph < 2 && r == hipSuccess; ++ph)
          r = psgd::launch_gs_bgemm(pass, kb, ph, dm, W(W_BGEMM) + plan->bg_off[kb][ph], plan->bg_cnt[kb][ph], stream);
      }
      return r; });
  } else {
    e = run(S_FACTOR, [&] { return psgd::launch_gs_factor(pass, dm, W(W_FACTOR), plan->cnt[W_FACTOR], stream); });
  }
  if (e != hipSuccess) return e;
  return run(S_APPLY, [&] { return psgd::launch_gs_apply(plan->rt, big, pass, dm, W(W_APPLY), plan->cnt[W_APPLY], stream); });
}
}  // namespace

psgd_status psgd_orthogonalize(psgd_ctx* ctx, psgd_plan* plan, hipStream_t stream) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  HIPCHK(ctx, orth_pass(plan, 0, stream, ctx, true), "orthonormalisation");
  // second pass, for the matrices whose first pass flagged it (the others return at once)
  HIPCHK(ctx, traced(ctx, S_REORTH, stream, [&] { return orth_pass(plan, 1, stream, ctx, false); }),
         "second orthonormalisation pass");
  return PSGD_OK;
}

psgd_status psgd_compress_q(psgd_ctx* ctx, psgd_plan* plan, const float* scale, hipStream_t stream) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  if (!scale) return fail(ctx, PSGD_EINVAL, "scale is required");
  const DevMat* dm = plan->d_mats;
  auto W = [&](int k) { return plan->d_work + plan->off[k]; };
  if (plan->big)
    HIPCHK(ctx, traced(ctx, S_K2, stream, [&] { return psgd::launch_gemm_nt(dm, W(W_G2), plan->cnt[W_G2], true, stream); }), "M^T P");
  else
    HIPCHK(ctx, traced(ctx, S_K2, stream, [&] { return psgd::launch_mtp(plan->gt, plan->rtc, dm, W(W_K2), plan->cnt[W_K2], scale, stream); }), "M^T P");
  if (plan->big)
    HIPCHK(ctx, traced(ctx, S_SPLIT3, stream, [&] { return psgd::launch_split3(dm, W(W_SPLIT3), plan->cnt[W_SPLIT3], stream); }), "decompression row scales");
  return PSGD_OK;
}

psgd_status psgd_refresh_q(psgd_ctx* ctx, psgd_plan* plan, hipStream_t stream) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  const DevMat* dm = plan->d_mats;
  auto W = [&](int k) { return plan->d_work + plan->off[k]; };
  HIPCHK(ctx, traced(ctx, S_SPLIT3, stream, [&] { return psgd::launch_split3(dm, W(W_SPLITQ), plan->cnt[W_SPLITQ], stream); }), "decompression row scales of q_next");
  return PSGD_OK;
}

psgd_status psgd_compress(psgd_ctx* ctx, psgd_plan* plan, const float* scale, uint8_t* flags,
                          hipStream_t stream) {
  if (psgd_status st = psgd_compress_p(ctx, plan, scale, flags, stream); st != PSGD_OK) return st;
  if (psgd_status st = psgd_orthogonalize(ctx, plan, stream); st != PSGD_OK) return st;
  return psgd_compress_q(ctx, plan, scale, stream);
}

psgd_status psgd_factor_buffer(psgd_plan* plan, void** ptr, int64_t* count, int32_t* rpad) {
  if (!plan || !ptr || !count) return PSGD_EINVAL;
  *ptr = plan->workspace;
  *count = (int64_t)(plan->praw_bytes / 4);
  if (rpad) *rpad = plan->mats.empty() ? 0 : plan->mats[0].rpad;
  return PSGD_OK;
}

psgd_status psgd_check_finite(psgd_ctx* ctx, psgd_plan* plan, const uint8_t* flags,
                              const psgd_tensor* pass, int n_pass, const float* scale,
                              int32_t* skip_dev, int32_t* skip_host, hipStream_t stream) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!plan || plan->ctx != ctx) return fail(ctx, PSGD_EINVAL, "plan does not belong to this context");
  if (!flags || !scale || !skip_dev) return fail(ctx, PSGD_EINVAL, "flags, scale and skip_dev are required");
  if (n_pass < 0 || (n_pass > 0 && !pass)) return fail(ctx, PSGD_EINVAL, "bad pass-through list");
  std::vector<const float*> ptrs;
  std::vector<int64_t> ns;
  for (int i = 0; i < n_pass; ++i) {
    if (pass[i].numel < 0 || (pass[i].numel > 0 && !pass[i].data))
      return fail(ctx, PSGD_EINVAL, "pass-through tensor %d: bad pointer or size", i);
    if (pass[i].numel == 0) continue;
    ptrs.push_back(pass[i].data);
    ns.push_back(pass[i].numel);
  }
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  HIPCHK(ctx, traced(ctx, S_ZERO_SKIP, stream, [&] { return psgd::launch_zero_i32(skip_dev, 1, stream); }), "skip clear");
  HIPCHK(ctx, traced(ctx, S_CHECK, stream, [&] {
                return psgd::launch_check_finite(flags, plan->n_mats, scale, plan->n_blocks, ptrs.data(),
                                                 ns.data(), (int)ptrs.size(), skip_dev, stream); }), "finite check");
  if (skip_host) {
    HIPCHK(ctx, hipMemcpyAsync(skip_host, skip_dev, sizeof(int32_t), hipMemcpyDeviceToHost, stream), "skip copy");
    HIPCHK(ctx, hipStreamSynchronize(stream), "skip sync");
  }
  return PSGD_OK;
}

psgd_status psgd_decompress_update(psgd_ctx* ctx, psgd_plan* plan, const float* scale,
                                   const int32_t* skip_dev, hipStream_t stream) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!plan || plan->ctx != ctx) return fail(ctx, PSGD_EINVAL, "plan does not belong to this context");
  if (!scale || !skip_dev) return fail(ctx, PSGD_EINVAL, "scale and skip_dev are required");
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  const DevMat* dm = plan->d_mats;
  auto W = [&](int k) { return plan->d_work + plan->off[k]; };
  HIPCHK(ctx, traced(ctx, S_K3, stream, [&] { return psgd::launch_decompress(plan->gt, plan->big, dm, W(W_K3), plan->cnt[W_K3], scale, skip_dev, plan->d_counters, stream); }), "decompress");
  return PSGD_OK;
}

psgd_status psgd_reset_errors(psgd_ctx* ctx, psgd_plan* plan, hipStream_t stream) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!plan || plan->ctx != ctx) return fail(ctx, PSGD_EINVAL, "plan does not belong to this context");
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  // the decompression's skipped form zeroes every error buffer and touches nothing else (no
  // scale is read on that path; the pointer only has to be valid)
  const float* any_scale = reinterpret_cast<const float*>(plan->d_one);
  HIPCHK(ctx, traced(ctx, S_K3, stream, [&] { return psgd::launch_decompress(plan->gt, plan->big, plan->d_mats, plan->d_work + plan->off[W_K3], plan->cnt[W_K3], any_scale, plan->d_one, nullptr, stream); }), "error buffer reset");
  return PSGD_OK;
}

namespace {
psgd_status check_block_args(psgd_ctx* ctx, const void* a, const void* b, int64_t n, const float* scale,
                             psgd_dtype dt) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (n < 0) return fail(ctx, PSGD_EINVAL, "negative element count");
  if (dt != PSGD_F16 && dt != PSGD_BF16) return fail(ctx, PSGD_EDTYPE, "the block's gradient type must be fp16 or bf16");
  if (n == 0) return PSGD_OK;
  if (!a || !b || !scale) return fail(ctx, PSGD_EINVAL, "NULL tensor or scale pointer");
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15)
    return fail(ctx, PSGD_EINVAL, "tensor base addresses must be 16-byte aligned");
  return PSGD_OK;
}
}  // namespace

psgd_status psgd_block_grad_enter(psgd_ctx* ctx, const float* dx, int64_t n, const float* scale,
                                  void* out, psgd_dtype out_dtype, hipStream_t stream) {
  if (psgd_status st = check_block_args(ctx, dx, out, n, scale, out_dtype); st != PSGD_OK || n == 0) return st;
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  HIPCHK(ctx, psgd::launch_block_enter(out_dtype == PSGD_F16 ? psgd::G_F16 : psgd::G_BF16, dx, n, scale,
                                       static_cast<uint16_t*>(out), stream), "block entry scaling");
  return PSGD_OK;
}

psgd_status psgd_block_grad_exit(psgd_ctx* ctx, float* dx, const void* g, int64_t n, const float* scale,
                                 psgd_dtype g_dtype, uint8_t* flag, hipStream_t stream) {
  if (psgd_status st = check_block_args(ctx, dx, g, n, scale, g_dtype); st != PSGD_OK || n == 0) return st;
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  HIPCHK(ctx, psgd::launch_block_exit(g_dtype == PSGD_F16 ? psgd::G_F16 : psgd::G_BF16, dx,
                                      static_cast<const uint16_t*>(g), n, scale, flag, stream), "block exit unscaling");
  return PSGD_OK;
}

psgd_status psgd_block_grad_exit_enter(psgd_ctx* ctx, float* dx, const void* g, int64_t n,
                                       const float* scale_exit, const float* scale_enter, void* out,
                                       psgd_dtype dtype, uint8_t* flag, hipStream_t stream) {
  if (psgd_status st = check_block_args(ctx, dx, g, n, scale_exit, dtype); st != PSGD_OK || n == 0) return st;
  if (!scale_enter || !out) return fail(ctx, PSGD_EINVAL, "NULL tensor or scale pointer");
  if (reinterpret_cast<uintptr_t>(out) & 15) return fail(ctx, PSGD_EINVAL, "tensor base addresses must be 16-byte aligned");
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  HIPCHK(ctx, psgd::launch_block_exit_enter(dtype == PSGD_F16 ? psgd::G_F16 : psgd::G_BF16, dx,
                                            static_cast<const uint16_t*>(g), n, scale_exit, scale_enter,
                                            static_cast<uint16_t*>(out), flag, stream), "block boundary rescaling");
  return PSGD_OK;
}

psgd_status psgd_step_noalloc(psgd_ctx* ctx, const psgd_matrix* mats, int n_mats,
                              psgd_dtype grad_dtype, const float* scale, int n_blocks,
                              const psgd_tensor* pass, int n_pass, uint8_t* flags,
                              int32_t* skip_dev, hipStream_t stream) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!scale || !flags || !skip_dev) return fail(ctx, PSGD_EINVAL, "scale, flags and skip_dev are required");
  if (!ctx->scratch) return fail(ctx, PSGD_EHIP, "no scratch array on device %d", ctx->device);
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  // Lay the group out exactly as psgd_plan_create does (same descriptors, same work lists, so
  // the same kernels compute the same results), then place it in the scratch array:
  // [workspace | descriptor table | work lists].
  psgd_plan* p = ctx->noalloc_plan.get();
  PlanLayout L;
  if (psgd_status st = plan_layout(ctx, mats, n_mats, grad_dtype, n_blocks, p, L); st != PSGD_OK) return st;
  const size_t mats_off = L.ws;
  const size_t work_off = mats_off + (size_t)rup((int64_t)(sizeof(DevMat) * n_mats), 256);
  const size_t total = work_off + (size_t)rup((int64_t)(sizeof(Work) * L.all.size()), 256);
  if (total > kScratchBytes)
    return fail(ctx, PSGD_EINVAL,
                "the group needs %zu bytes of workspace; the allocation-free step holds at most %zu "
                "(use psgd_plan_create)", total, kScratchBytes);
  char* base = ctx->scratch;
  plan_bind(p, base, L);
  p->d_mats = reinterpret_cast<DevMat*>(base + mats_off);
  p->d_work = reinterpret_cast<Work*>(base + work_off);
  // The array keeps the previous call's contents: the workspace padding must read zero (it is
  // never written by the kernels), so the whole workspace is cleared first. Every step runs on
  // `stream`, in order; only kernels are launched (the uploads travel as kernel arguments).
  HIPCHK(ctx, psgd::launch_fill_zero(base, L.ws, stream), "scratch clear");
  const int32_t one = 1;
  HIPCHK(ctx, psgd::launch_upload(p->d_one, &one, sizeof one, stream), "constant upload");
  HIPCHK(ctx, psgd::launch_upload(p->d_mats, p->mats.data(), sizeof(DevMat) * n_mats, stream), "descriptor upload");
  HIPCHK(ctx, psgd::launch_upload(p->d_work, L.all.data(), sizeof(Work) * L.all.size(), stream), "work list upload");
  if (psgd_status st = psgd_compress(ctx, p, scale, flags, stream); st != PSGD_OK) return st;
  if (psgd_status st = psgd_check_finite(ctx, p, flags, pass, n_pass, scale, skip_dev, nullptr, stream); st != PSGD_OK)
    return st;
  return psgd_decompress_update(ctx, p, scale, skip_dev, stream);
}

// ------------------------------------------------------------------------------------------
// the optimizer step that consumes the decompressed gradient
// ------------------------------------------------------------------------------------------
psgd_status psgd_adam_attach(psgd_ctx* ctx, psgd_plan* plan, const psgd_adam_matrix* opt,
                             psgd_dtype param_dtype) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  if (!opt) return fail(ctx, PSGD_EINVAL, "optimizer descriptors are required");
  int pt = 0, psz = 0;
  switch (param_dtype) {
    case PSGD_F16: pt = psgd::G_F16; psz = 2; break;
    case PSGD_BF16: pt = psgd::G_BF16; psz = 2; break;
    case PSGD_F32: pt = psgd::G_F32; psz = 4; break;
    default: return fail(ctx, PSGD_EDTYPE, "unknown parameter dtype %d", (int)param_dtype);
  }
  std::vector<DevMat> mats = plan->mats;
  std::vector<psgd::NormItem> items;
  for (int i = 0; i < plan->n_mats; ++i) {
    const psgd_adam_matrix& a = opt[i];
    DevMat& d = mats[i];
    if (!a.param || !a.m1 || !a.m2) return fail(ctx, PSGD_EINVAL, "matrix %d: param, m1 and m2 are required", i);
    if (!aligned16(a.param) || !aligned16(a.m1) || !aligned16(a.m2))
      return fail(ctx, PSGD_EINVAL, "matrix %d: param, m1 and m2 must be 16-byte aligned", i);
    if (a.ld_param < d.n || a.ld_param % 8 != 0)
      return fail(ctx, PSGD_EINVAL, "matrix %d: ld_param must be >= n and a multiple of 8", i);
    const int64_t pb = ((int64_t)(d.m - 1) * a.ld_param + d.n) * psz;
    const int64_t mb = (int64_t)d.m * d.n * 2;
    if (pb >= (int64_t(1) << 31) || mb >= (int64_t(1) << 31))
      return fail(ctx, PSGD_EINVAL, "matrix %d: param and moments must each span less than 2 GiB", i);
    d.param = a.param;
    d.ld_param = a.ld_param;
    d.m1 = a.m1;
    d.m2 = a.m2;
    d.p_bytes = (uint32_t)pb;
    d.mo_bytes = (uint32_t)mb;
    // the norm of D is that of q_next (n x r): items of at most kNormItem floats
    const int64_t cnt = (int64_t)d.n * d.r;
    for (int64_t o = 0; o < cnt; o += psgd::kNormItem)
      items.push_back(psgd::NormItem{d.q_next + o, std::min<int64_t>(psgd::kNormItem, cnt - o)});
  }
  const size_t items_bytes = (size_t)rup((int64_t)((items.size() + kMaxPassItems) * sizeof(psgd::NormItem)), 256);
  const size_t bytes = items_bytes + (items.size() + kMaxPassItems) * sizeof(double);
  void* buf = nullptr;
  hipError_t e = hipDeviceSynchronize();        // no step of this plan may still be running
  if (e != hipSuccess) return hip_fail(ctx, e, "synchronise before attaching");
  if ((e = hipMalloc(&buf, bytes)) != hipSuccess) return fail(ctx, PSGD_ENOMEM, "optimizer buffer of %zu bytes", bytes);
  if ((e = hipMemcpy(buf, items.data(), items.size() * sizeof(psgd::NormItem), hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(plan->d_mats, mats.data(), sizeof(DevMat) * plan->n_mats, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipDeviceSynchronize()) != hipSuccess) {
    (void)hipFree(buf);
    return hip_fail(ctx, e, "optimizer upload");
  }
  if (plan->adam_buf) (void)hipFree(plan->adam_buf);
  plan->mats = mats;
  plan->adam_buf = buf;
  plan->d_items = static_cast<psgd::NormItem*>(buf);
  plan->d_partial = reinterpret_cast<double*>(static_cast<char*>(buf) + items_bytes);
  plan->n_plan_items = (int)items.size();
  plan->adam_pt = pt;
  return PSGD_OK;
}

namespace {
psgd_status check_pass_tensors(psgd_ctx* ctx, const psgd_adam_tensor* pass, int n_pass, bool update) {
  if (n_pass < 0 || (n_pass > 0 && !pass)) return fail(ctx, PSGD_EINVAL, "bad pass-through list");
  for (int i = 0; i < n_pass; ++i) {
    const psgd_adam_tensor& t = pass[i];
    if (t.numel < 0) return fail(ctx, PSGD_EINVAL, "pass-through tensor %d: negative size", i);
    if (t.numel == 0) continue;
    if (!t.grad || (update && (!t.param || !t.m1 || !t.m2)))
      return fail(ctx, PSGD_EINVAL, "pass-through tensor %d: NULL pointer", i);
  }
  return PSGD_OK;
}
psgd::AdamArgs adam_args(const psgd_adam_hparams* hp, const int32_t* step, const float* norm) {
  return psgd::AdamArgs{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, step, norm + 1};
}
psgd_status check_hparams(psgd_ctx* ctx, const psgd_adam_hparams* hp) {
  if (!hp) return fail(ctx, PSGD_EINVAL, "hyperparameters are required");
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return fail(ctx, PSGD_EINVAL, "betas must lie in [0, 1)");
  if (!(hp->eps >= 0.0f) || !(hp->lr >= 0.0f) || !(hp->weight_decay >= 0.0f) ||
      !std::isfinite(hp->eps) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
    return fail(ctx, PSGD_EINVAL, "lr, eps and weight_decay must be finite and >= 0");
  return PSGD_OK;
}
}  // namespace

psgd_status psgd_adam_prepare(psgd_ctx* ctx, psgd_plan* plan, const psgd_adam_tensor* pass, int n_pass,
                              float max_norm, const int32_t* skip_dev, int32_t* step_dev,
                              float* norm_dev, hipStream_t stream) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  if (!plan->adam_pt) return fail(ctx, PSGD_EINVAL, "no optimizer attached to the plan (psgd_adam_attach)");
  if (!skip_dev || !step_dev || !norm_dev) return fail(ctx, PSGD_EINVAL, "skip_dev, step_dev and norm_dev are required");
  if (psgd_status st = check_pass_tensors(ctx, pass, n_pass, false); st != PSGD_OK) return st;
  std::vector<psgd::NormItem> items;
  for (int i = 0; i < n_pass; ++i)
    for (int64_t o = 0; o < pass[i].numel; o += psgd::kNormItem)
      items.push_back(psgd::NormItem{pass[i].grad + o, std::min<int64_t>(psgd::kNormItem, pass[i].numel - o)});
  if ((int)items.size() > kMaxPassItems)
    return fail(ctx, PSGD_EINVAL, "pass-through gradients hold more than %lld elements",
                (long long)kMaxPassItems * psgd::kNormItem);
  const int n_items = plan->n_plan_items + (int)items.size();
  HIPCHK(ctx, traced(ctx, S_ADAM_NORM, stream, [&] {
    hipError_t e = items.empty() ? hipSuccess
                                 : psgd::launch_upload(plan->d_items + plan->n_plan_items, items.data(),
                                                       items.size() * sizeof(psgd::NormItem), stream);
    if (e == hipSuccess) e = psgd::launch_sqnorm(plan->d_items, n_items, plan->d_partial, stream);
    if (e == hipSuccess) e = psgd::launch_adam_finalize(plan->d_partial, n_items, max_norm, skip_dev, step_dev,
                                                        norm_dev, stream);
    return e; }), "global gradient norm");
  return PSGD_OK;
}

psgd_status psgd_decompress_adam(psgd_ctx* ctx, psgd_plan* plan, const float* scale, const int32_t* skip_dev,
                                 const int32_t* step_dev, const float* norm_dev,
                                 const psgd_adam_hparams* hp, hipStream_t stream) {
  if (psgd_status st = check_call(ctx, plan); st != PSGD_OK) return st;
  if (!plan->adam_pt) return fail(ctx, PSGD_EINVAL, "no optimizer attached to the plan (psgd_adam_attach)");
  if (!scale || !skip_dev || !step_dev || !norm_dev) return fail(ctx, PSGD_EINVAL, "scale, skip_dev, step_dev and norm_dev are required");
  if (psgd_status st = check_hparams(ctx, hp); st != PSGD_OK) return st;
  const psgd::AdamArgs aa = adam_args(hp, step_dev, norm_dev);
  HIPCHK(ctx, traced(ctx, S_K3_ADAM, stream, [&] {
    return psgd::launch_decompress_adam(plan->gt, plan->adam_pt, plan->big, plan->d_mats, plan->d_work + plan->off[W_K3],
                                        plan->cnt[W_K3], scale, skip_dev, aa, plan->d_counters, stream); }), "decompression with Adam");
  return PSGD_OK;
}

psgd_status psgd_adam_update(psgd_ctx* ctx, const psgd_adam_tensor* pass, int n_pass, const int32_t* skip_dev,
                             const int32_t* step_dev, const float* norm_dev, const psgd_adam_hparams* hp,
                             hipStream_t stream) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!skip_dev || !step_dev || !norm_dev) return fail(ctx, PSGD_EINVAL, "skip_dev, step_dev and norm_dev are required");
  if (psgd_status st = check_hparams(ctx, hp); st != PSGD_OK) return st;
  if (psgd_status st = check_pass_tensors(ctx, pass, n_pass, true); st != PSGD_OK) return st;
  std::vector<psgd::AdamTensor> ts;
  for (int i = 0; i < n_pass; ++i)
    if (pass[i].numel > 0)
      ts.push_back(psgd::AdamTensor{pass[i].param, pass[i].m1, pass[i].m2, pass[i].grad, pass[i].numel});
  HIPCHK(ctx, hipSetDevice(ctx->device), "hipSetDevice");
  const psgd::AdamArgs aa = adam_args(hp, step_dev, norm_dev);
  HIPCHK(ctx, traced(ctx, S_ADAM_PASS, stream, [&] {
    return psgd::launch_adam_f32(ts.data(), (int)ts.size(), aa, skip_dev, stream); }), "pass-through Adam");
  return PSGD_OK;
}

psgd_status psgd_profile_events(psgd_ctx* ctx, hipEvent_t* events, int n) {
  if (!ctx) return PSGD_EINVAL;
  ctx->err.clear();
  if (!events) {
    ctx->events.clear();
    return PSGD_OK;
  }
  if (n < 2 * S_SLOTS) return fail(ctx, PSGD_EINVAL, "need at least %d events, got %d", 2 * S_SLOTS, n);
  ctx->events.assign(events, events + 2 * S_SLOTS);
  return PSGD_OK;
}

psgd_status psgd_plan_counters(psgd_plan* plan, const int64_t** counters) {
  if (!plan || !counters) return PSGD_EINVAL;
  *counters = plan->d_counters;
  return PSGD_OK;
}

psgd_status psgd_debug_buffer(psgd_plan* plan, int which, int mat, void** ptr, int64_t* bytes,
                              int32_t* rpad) {
  if (!plan || !ptr || !bytes || mat < 0 || mat >= plan->n_mats) return PSGD_EINVAL;
  const DevMat& d = plan->mats[mat];
  if (rpad) *rpad = d.rpad;
  switch (which) {
    case 0: *ptr = d.p_raw; *bytes = (int64_t)d.m * d.rpad * 4; return PSGD_OK;
    case 1: *ptr = d.tmat; *bytes = (int64_t)d.rpad * d.rpad * 8; return PSGD_OK;
  }
  return PSGD_EINVAL;
}

}  // extern "C"
