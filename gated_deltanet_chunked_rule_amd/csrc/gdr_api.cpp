// gdr_api.cpp -- C ABI of libgdr: argument validation, the host planner
// (chunk counts, the context-parallel split), workspace layout and the
// launch sequence.  See include/gdr.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdr.h"
#include "gdr_kernels.h"

// Workspace of gdr_chunk_fwd_noalloc: device memory owned by the library, one
// copy per device (each device that loads the library holds it until the
// process ends).  Host code never uses this name as an address: it is a
// host-side stand-in; the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string t_err;

gdr_status fail(gdr_status s, const std::string& msg) {
  t_err = msg;
  return s;
}

constexpr int kChunk = 64;
constexpr int kMaxOrderedSegs = 1024;   // segments the plan kernel ranks for the dispatch order
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kStateWgPerCU = 1;   // fused state workgroups (8 waves) resident per CU
constexpr size_t kAlign = 256;

struct Problem {
  int B = 0, T = 0, Hq = 0, Hv = 0, K = 0, V = 0, N = 0;
  gdr::DType dt = gdr::DType::BF16;
  size_t esize = 2;
  long Ttot = 0;
  bool packed = false;
  std::vector<int> chunks;  // per sequence
  int NTtot = 0, NTmax = 0;
  // plan
  int BV = 0, nvb = 0, L = 1, W = 0, total_segs = 0;
  float log_eps = 0.f;
  bool serial_fallback = false;   // uncertified heads run serially instead of exact segments
  bool precise_vnew = false;      // bf16 output pass with Vnew as two bf16 terms
};

struct Layout {
  size_t cu = 0, chunk_off = 0, seg_off = 0, gcum = 0, cert = 0, W = 0, U = 0, vnew = 0, hbuf = 0;
  size_t A = 0, dhbuf = 0, dvn = 0, segtr = 0, hstart = 0, Au = 0, seg_order = 0, hflag = 0, total = 0;
};

// bf16 stages A diag(beta) per chunk and V, and forms Vnew (and, in the
// backward's reverse pass, W^T dVnew) from them, instead of a W and U round
// trip through HBM; fp32 keeps W and U.
bool apath(const Problem& P) { return P.dt == gdr::DType::BF16; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Segment length (chunks) for the serial state pass.  Each (sequence, value
// head, V block) is one serial unit of work; when those units cannot fill the
// GPU, sequences are cut into segments of L chunks, each preceded by W warmup
// chunks.  L minimises max(critical path, total steps / resident slots): the
// segment count is what fills the GPU, the reading of the pages' "choose L
// proportional to N" rule (FlashQLA curated summary, section
// "平衡解決方案：雙核心融合與自動CP").  The page's H200 trigger thresholds are not
// reused: they describe a 132-SM part.
int choose_segment(const Problem& P) {
  const int W = P.W;
  const long slots = (long)kCUs * kStateWgPerCU;
  const long units = (long)P.Hv;     // the fused pass covers all V columns per workgroup
  const int NTmax = std::max(P.NTmax, 1);
  const long base = units * (long)P.N;
  if (base >= slots || NTmax <= 2 * W + 1) return NTmax;
  auto cost = [&](int L) {
    double total = 0.0;
    int crit = 0;
    for (int c : P.chunks) {
      const int segs = std::max(1, (c + L - 1) / L);
      long steps = c;
      for (int s = 1; s < segs; ++s) steps += std::min(W, s * L);
      total += (double)units * steps;
      crit = std::max(crit, segs > 1 ? std::min(L, c) + W : c);
    }
    return std::max((double)crit, total / (double)slots);
  };
  int best = NTmax;
  double best_cost = cost(NTmax);
  static const int parts[] = {2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32, 40, 48, 64, 80, 96, 128,
                              160, 192, 256, 320, 384, 512, 768, 1024};
  for (int pc : parts) {
    const int L = (NTmax + pc - 1) / pc;
    if (L < 1) break;
    const double c = cost(L);
    if (c < best_cost * 0.98) {  // prefer fewer segments unless clearly faster
      best_cost = c;
      best = L;
    }
  }
  return best;
}

gdr_status analyze(const gdr_shape* sh, const gdr_options* op, const int32_t* cu_host,
                   bool packed, Problem& P) {
  if (!sh) return fail(GDR_ERR_INVALID_ARG, "shape is NULL");
  P.B = sh->B; P.T = sh->T; P.Hq = sh->Hq; P.Hv = sh->Hv; P.K = sh->K; P.V = sh->V;
  if (P.B < 1 || P.T < 0 || P.Hq < 1 || P.Hv < 1 || P.K < 1 || P.V < 1)
    return fail(GDR_ERR_INVALID_ARG, "shape dimensions must be positive (T may be 0)");
  if (P.Hv % P.Hq != 0) return fail(GDR_ERR_INVALID_ARG, "Hv must be a multiple of Hq");
  if ((long)P.B * P.T > 0x7fffffffL) return fail(GDR_ERR_UNSUPPORTED, "B*T exceeds 2^31-1 tokens");
  if (sh->dtype == GDR_BF16) { P.dt = gdr::DType::BF16; P.esize = 2; }
  else if (sh->dtype == GDR_F32) { P.dt = gdr::DType::F32; P.esize = 4; }
  else return fail(GDR_ERR_UNSUPPORTED, "dtype must be GDR_BF16 or GDR_F32");
  if (P.K != P.V) return fail(GDR_ERR_UNSUPPORTED, "K must equal V");
  if (P.K != 32 && P.K != 64 && P.K != 128) return fail(GDR_ERR_UNSUPPORTED, "K must be 32, 64 or 128");
  if (P.dt == gdr::DType::F32 && P.K > 64) return fail(GDR_ERR_UNSUPPORTED, "fp32 supports K <= 64");
  P.Ttot = (long)P.B * P.T;
  P.packed = packed;
  if (packed) {
    if (!cu_host) return fail(GDR_ERR_INVALID_ARG, "packed mode needs cu_seqlens_host");
    if (P.B != 1) return fail(GDR_ERR_INVALID_ARG, "packed mode (cu_seqlens) requires B == 1");
    P.N = sh->num_seqs;
    if (P.N < 1) return fail(GDR_ERR_INVALID_ARG, "num_seqs must be >= 1 in packed mode");
    if (cu_host[0] != 0) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
    for (int n = 0; n < P.N; ++n)
      if (cu_host[n + 1] < cu_host[n]) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
    if (cu_host[P.N] != P.T) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens[num_seqs] must equal T");
  } else {
    P.N = P.B;
  }
  P.chunks.resize(P.N);
  P.NTtot = 0;
  P.NTmax = 0;
  for (int n = 0; n < P.N; ++n) {
    const int len = packed ? cu_host[n + 1] - cu_host[n] : P.T;
    const int c = (len + kChunk - 1) / kChunk;
    P.chunks[n] = c;
    P.NTtot += c;
    P.NTmax = std::max(P.NTmax, c);
  }
  // options
  gdr_cp_mode mode = GDR_CP_AUTO;
  int forced = 0;
  P.W = 8;
  P.log_eps = std::log(1e-6f);
  if (op) {
    mode = op->cp_mode;
    forced = op->cp_segment_chunks;
    if (op->cp_warmup_chunks > 0) P.W = op->cp_warmup_chunks;
    else if (op->cp_warmup_chunks < 0) return fail(GDR_ERR_INVALID_ARG, "cp_warmup_chunks must be >= 0");
    if (op->cp_log_eps != 0.f) P.log_eps = op->cp_log_eps;
    if (!(P.log_eps < 0.f)) return fail(GDR_ERR_INVALID_ARG, "cp_log_eps must be negative");
    if (op->cp_serial_fallback != 0 && op->cp_serial_fallback != 1)
      return fail(GDR_ERR_INVALID_ARG, "cp_serial_fallback must be 0 or 1");
    P.serial_fallback = op->cp_serial_fallback == 1;
    if (op->precise_vnew != 0 && op->precise_vnew != 1) return fail(GDR_ERR_INVALID_ARG, "precise_vnew must be 0 or 1");
    P.precise_vnew = op->precise_vnew == 1;
  }
  P.BV = (P.K == 128) ? 64 : 32;
  P.nvb = P.V / P.BV;
  const int NTmax1 = std::max(P.NTmax, 1);
  if (mode == GDR_CP_OFF) {
    P.L = NTmax1;
  } else if (mode == GDR_CP_FORCE) {
    if (forced < 1) return fail(GDR_ERR_INVALID_ARG, "GDR_CP_FORCE needs cp_segment_chunks >= 1");
    P.L = std::min(forced, NTmax1);
  } else if (mode == GDR_CP_AUTO) {
    P.L = choose_segment(P);
  } else {
    return fail(GDR_ERR_INVALID_ARG, "unknown cp_mode");
  }
  P.total_segs = 0;
  for (int c : P.chunks) P.total_segs += std::max(1, (c + P.L - 1) / P.L);
  return GDR_OK;
}

// CP segments (forward, and the bf16 backward): heads that fail the warmup
// certificate get exact segment start states (transition pass + scan) unless
// the caller asked for the serial fallback.
bool exact_cp(const Problem& P, int L) { return L < P.NTmax && !P.serial_fallback; }
bool exact_cp(const Problem& P) { return exact_cp(P, P.L); }
// The bf16 backward runs its serial passes in CP segments; fp32 runs them whole.
bool bwd_segmented(const Problem& P) { return P.dt == gdr::DType::BF16; }

Layout layout(const Problem& P, bool bwd) {
  Layout Lo;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t nn = (size_t)P.N + 1, hv = (size_t)P.Hv, tt = (size_t)P.Ttot, nt = (size_t)P.NTtot;
  Lo.cu = take(nn * 4);
  Lo.chunk_off = take(nn * 4);
  Lo.seg_off = take(nn * 4);
  Lo.seg_order = take(kMaxOrderedSegs * 4);
  Lo.gcum = take(hv * tt * 4);
  Lo.cert = take(hv * nt * 4);
  Lo.hflag = take(nn * hv * 4);
  if (apath(P)) {
    Lo.Au = take(hv * tt * kChunk * 2);
  } else {
    Lo.W = take(hv * tt * P.K * P.esize);
    Lo.U = take(hv * tt * P.V * P.esize);
  }
  if (bwd) {
    Lo.vnew = take(hv * tt * P.V * P.esize);
    Lo.hbuf = take(hv * nt * P.V * P.K * P.esize);
    Lo.A = take(hv * tt * kChunk * 4);
    Lo.dhbuf = take(hv * nt * P.V * P.K * P.esize);
    Lo.dvn = take(hv * tt * P.V * P.esize);
  }
  if (exact_cp(P) && (!bwd || bwd_segmented(P))) {
    const size_t segs = (size_t)P.total_segs, kv = (size_t)P.K * P.V * 4;
    Lo.segtr = take(hv * segs * 2 * kv);
    Lo.hstart = take(hv * segs * kv);
  }
  Lo.total = off;
  return Lo;
}

// Packed batches of unequal sequences dispatch their state segments longest
// first (ranked on the device by k_plan, at most kMaxOrderedSegs of them): the
// number of segments for segment length L, or 0 when no order is used.
int ordered_segs(const Problem& P, int L) {
  if (!P.packed || P.chunks.empty()) return 0;
  int segs = 0;
  bool equal = true;
  for (int c : P.chunks) {
    segs += std::max(1, (c + std::max(L, 1) - 1) / std::max(L, 1));
    equal = equal && c == P.chunks[0];
  }
  return (equal || segs > kMaxOrderedSegs) ? 0 : segs;
}

// L: the CP segment length of the passes that read the segment offsets.
gdr::SeqTables tables(const Problem& P, const Layout& Lo, char* ws, int L) {
  gdr::SeqTables s;
  s.cu = reinterpret_cast<const int32_t*>(ws + Lo.cu);
  s.chunk_off = reinterpret_cast<const int32_t*>(ws + Lo.chunk_off);
  s.seg_off = reinterpret_cast<const int32_t*>(ws + Lo.seg_off);
  s.N = P.N;
  s.Ttot = P.Ttot;
  s.NTtot = P.NTtot;
  s.T_uniform = P.packed ? 0 : P.T;
  const int ntu = (P.T + kChunk - 1) / kChunk;
  s.segs_uniform = std::max(1, (ntu + std::max(L, 1) - 1) / std::max(L, 1));
  const int segs = ordered_segs(P, L);
  s.seg_order = segs > 0 ? reinterpret_cast<const int32_t*>(ws + Lo.seg_order) : nullptr;
  return s;
}

gdr_status hip_fail(hipError_t e, const char* what) {
  return fail(GDR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Plan tables + the forward chain: intra-chunk WY, then either the fused
// state+output pass (forward) or the state pass storing every chunk's entry
// state (backward recompute).
gdr_status run_forward_chain(const Problem& P, const Layout& Lo, char* ws, const void* q,
                             const void* k, const void* v, const float* g, const float* beta,
                             float scale, const float* h0, const int32_t* cu_dev, void* o,
                             float* ht, float* g_cum_out, float* A_out, float* A_ws, void* A_bf,
                             const float* A_in, int L, bool bwd, hipStream_t st) {
  hipError_t e;
  gdr::PlanParams pp;
  pp.cu_in = cu_dev;
  pp.N = P.N;
  pp.T = P.T;
  pp.seg_chunks = L;
  pp.cu = reinterpret_cast<int32_t*>(ws + Lo.cu);
  pp.chunk_off = reinterpret_cast<int32_t*>(ws + Lo.chunk_off);
  pp.seg_off = reinterpret_cast<int32_t*>(ws + Lo.seg_off);
  const gdr::SeqTables s = tables(P, Lo, ws, L);
  pp.seg_order = const_cast<int32_t*>(s.seg_order);
  pp.total_segs = ordered_segs(P, L);
  pp.warmup = P.W;
  // uniform rows need no tables: every kernel derives them arithmetically
  if (s.T_uniform <= 0 && (e = gdr::launch_plan(pp, st)) != hipSuccess) return hip_fail(e, "plan launch");
  if (P.NTtot > 0) {
    gdr::IntraParams ip;
    ip.s = s; ip.k = k; ip.v = v; ip.g = g; ip.beta = beta; ip.Hq = P.Hq; ip.Hv = P.Hv;
    ip.gcum = reinterpret_cast<float*>(ws + Lo.gcum);
    ip.g_cum_out = g_cum_out;
    ip.cert = reinterpret_cast<float*>(ws + Lo.cert);
    const bool ap = apath(P);
    ip.W = ap ? nullptr : ws + Lo.W; ip.U = ap ? nullptr : ws + Lo.U;
    ip.Au = ap ? ws + Lo.Au : nullptr;
    ip.A_ws = A_ws; ip.A_bf = A_bf; ip.A_out = A_out; ip.A_in = A_in;
    if ((e = gdr::launch_intra(P.dt, P.K, ip, st)) != hipSuccess) return hip_fail(e, "intra launch");
  }
  int segs = 0;
  for (int c : P.chunks) segs += std::max(1, (c + L - 1) / L);
  if (!bwd || bwd_segmented(P)) {
    // forward: state recurrence fused with the output; backward recompute:
    // the same pass storing every chunk's entry state and Vnew instead
    gdr::FusedParams fp;
    fp.s = s; fp.q = q; fp.k = k; fp.W = ws + Lo.W; fp.U = ws + Lo.U;
    fp.v = v; fp.Au = apath(P) ? ws + Lo.Au : nullptr;
    fp.gcum = reinterpret_cast<const float*>(ws + Lo.gcum);
    fp.cert = reinterpret_cast<const float*>(ws + Lo.cert);
    fp.h0 = h0; fp.ht = ht; fp.o = o;
    fp.Hq = P.Hq; fp.Hv = P.Hv; fp.seg_chunks = L; fp.warmup = P.W; fp.total_segs = segs;
    fp.log_eps = P.log_eps; fp.scale = scale;
    fp.trans = 0; fp.segtr = nullptr; fp.hstart = nullptr;
    fp.rev_cert = bwd ? 1 : 0;
    fp.split_vnew = (!bwd && P.precise_vnew) ? 1 : 0;
    fp.hbuf = bwd ? ws + Lo.hbuf : nullptr;
    fp.vnew = bwd ? ws + Lo.vnew : nullptr;
    fp.hflag = nullptr;
    if (exact_cp(P, L)) {
      // transitions (M, b) of the uncertified heads' segments, then their
      // exact start states; the transition pass records each head's
      // certificate decision for the scan and the output pass
      gdr::FusedParams tp = fp;
      tp.trans = 1;
      tp.hflag = reinterpret_cast<int*>(ws + Lo.hflag);
      tp.segtr = reinterpret_cast<float*>(ws + Lo.segtr);
      if ((e = gdr::launch_fused(P.dt, P.K, tp, segs, st)) != hipSuccess) return hip_fail(e, "transition launch");
      gdr::ScanParams sc;
      sc.s = s; sc.cert = fp.cert; sc.segtr = tp.segtr;
      sc.hstart = reinterpret_cast<float*>(ws + Lo.hstart);
      sc.Hv = P.Hv; sc.seg_chunks = L; sc.warmup = P.W; sc.total_segs = segs; sc.log_eps = P.log_eps;
      sc.rev = 0; sc.rev_cert = fp.rev_cert;
      sc.hflag = tp.hflag;
      if ((e = gdr::launch_segscan(P.K, sc, P.N * P.Hv, st)) != hipSuccess) return hip_fail(e, "scan launch");
      fp.hstart = sc.hstart;
      fp.hflag = tp.hflag;
    }
    if ((e = gdr::launch_fused(P.dt, P.K, fp, segs, st)) != hipSuccess) return hip_fail(e, "fused launch");
  } else {
    // backward recompute: every chunk's entry state and Vnew, row layouts
    gdr::StateParams sp;
    sp.s = s; sp.k = k; sp.W = ws + Lo.W; sp.U = ws + Lo.U;
    sp.gcum = reinterpret_cast<const float*>(ws + Lo.gcum);
    sp.cert = reinterpret_cast<const float*>(ws + Lo.cert);
    sp.h0 = h0; sp.ht = ht; sp.hbuf = ws + Lo.hbuf; sp.vnew = ws + Lo.vnew;
    sp.Hq = P.Hq; sp.Hv = P.Hv; sp.seg_chunks = L; sp.warmup = P.W; sp.log_eps = P.log_eps;
    sp.nvb = P.nvb;
    if ((e = gdr::launch_state(P.dt, P.K, P.BV, sp, segs, true, st)) != hipSuccess) return hip_fail(e, "state launch");
  }
  return GDR_OK;
}

// Device address of `scratch` on each device, looked up once per device (with
// that device current) on the first gdr_chunk_fwd_noalloc call there.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

gdr_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ERR_UNSUPPORTED, "device index beyond the scratch table");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p) return fail(GDR_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GDR_OK;
}

}  // namespace

extern "C" {

const char* gdr_last_error(void) { return t_err.c_str(); }

size_t gdr_chunk_fwd_workspace_size(const gdr_shape* shape, const gdr_options* opts,
                                    const int32_t* cu_seqlens_host) {
  Problem P;
  if (analyze(shape, opts, cu_seqlens_host, cu_seqlens_host != nullptr, P) != GDR_OK) return 0;
  return layout(P, false).total;
}

size_t gdr_chunk_bwd_workspace_size(const gdr_shape* shape, const gdr_options* opts,
                                    const int32_t* cu_seqlens_host) {
  Problem P;
  if (analyze(shape, opts, cu_seqlens_host, cu_seqlens_host != nullptr, P) != GDR_OK) return 0;
  if (P.dt == gdr::DType::F32 && P.K > 32) {
    fail(GDR_ERR_UNSUPPORTED, "fp32 backward supports K == 32");
    return 0;
  }
  return layout(P, true).total;
}

gdr_status gdr_chunk_fwd_plan(const gdr_shape* shape, const gdr_options* opts,
                              const int32_t* cu_seqlens_host, gdr_plan_info* out) {
  Problem P;
  gdr_status st = analyze(shape, opts, cu_seqlens_host, cu_seqlens_host != nullptr, P);
  if (st != GDR_OK) return st;
  if (!out) return fail(GDR_ERR_INVALID_ARG, "out is NULL");
  out->num_seqs = P.N;
  out->total_chunks = P.NTtot;
  out->max_chunks = P.NTmax;
  out->v_blocks = 1;
  out->segment_chunks = P.L;
  out->warmup_chunks = (P.L < P.NTmax) ? P.W : 0;
  out->total_segments = P.total_segs;
  out->state_workgroups = P.total_segs * P.Hv;
  return GDR_OK;
}

gdr_status gdr_chunk_fwd(const gdr_shape* shape, const gdr_options* opts, const void* q,
                         const void* k, const void* v, const float* g, const float* beta,
                         float scale, const float* initial_state, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, void* o, float* final_state,
                         float* g_cum_out, float* A_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (cu_seqlens_host && !cu_seqlens)
    return fail(GDR_ERR_INVALID_ARG, "cu_seqlens_host given without cu_seqlens");
  Problem P;
  gdr_status st = analyze(shape, opts, cu_seqlens_host, cu_seqlens != nullptr, P);
  if (st != GDR_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(GDR_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (P.Ttot > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, g, beta and o must be non-NULL");
  const void* ptrs[] = {q, k, v, g, beta, o, initial_state, cu_seqlens, final_state, g_cum_out, A_out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const Layout Lo = layout(P, false);
  if (!workspace || workspace_bytes < Lo.total)
    return fail(GDR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(Lo.total) + " bytes");
  char* ws = static_cast<char*>(workspace);
  return run_forward_chain(P, Lo, ws, q, k, v, g, beta, scale, initial_state, cu_seqlens, o,
                           final_state, g_cum_out, A_out, nullptr, nullptr, nullptr, P.L, false,
                           static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_fwd_noalloc(const gdr_shape* shape, const gdr_options* opts, const void* q,
                                 const void* k, const void* v, const float* g, const float* beta,
                                 float scale, const float* initial_state, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, void* o, float* final_state,
                                 float* g_cum_out, float* A_out, void* stream) {
  if (cu_seqlens_host && !cu_seqlens)
    return fail(GDR_ERR_INVALID_ARG, "cu_seqlens_host given without cu_seqlens");
  Problem P;
  gdr_status st = analyze(shape, opts, cu_seqlens_host, cu_seqlens != nullptr, P);
  if (st != GDR_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(GDR_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (P.Ttot > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, g, beta and o must be non-NULL");
  const void* ptrs[] = {q, k, v, g, beta, o, initial_state, cu_seqlens, final_state, g_cum_out, A_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const Layout Lo = layout(P, false);
  if (Lo.total > (size_t)GDR_NOALLOC_SCRATCH_BYTES)
    return fail(GDR_ERR_WORKSPACE, "problem needs " + std::to_string(Lo.total) +
                                       " bytes of workspace, beyond the library scratch of " +
                                       std::to_string((size_t)GDR_NOALLOC_SCRATCH_BYTES) +
                                       " bytes: use gdr_chunk_fwd with a caller workspace");
  // Every workspace element the forward reads is written by an earlier kernel
  // of the same call (nothing needs clearing), so the scratch's previous
  // contents do not matter.
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != GDR_OK) return st;
  return run_forward_chain(P, Lo, static_cast<char*>(ws), q, k, v, g, beta, scale, initial_state,
                           cu_seqlens, o, final_state, g_cum_out, A_out, nullptr, nullptr, nullptr, P.L,
                           false, static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_bwd(const gdr_shape* shape, const gdr_options* opts, const void* q,
                         const void* k, const void* v, const float* g, const float* beta,
                         const float* A, const void* d_o, const float* dht, float scale,
                         const float* initial_state, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, void* dq, void* dk, void* dv,
                         float* dbeta, float* dg, float* dh0, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (cu_seqlens_host && !cu_seqlens)
    return fail(GDR_ERR_INVALID_ARG, "cu_seqlens_host given without cu_seqlens");
  Problem P;
  gdr_status st = analyze(shape, opts, cu_seqlens_host, cu_seqlens != nullptr, P);
  if (st != GDR_OK) return st;
  if (P.dt == gdr::DType::F32 && P.K > 32) return fail(GDR_ERR_UNSUPPORTED, "fp32 backward supports K == 32");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(GDR_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (P.Ttot > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dbeta || !dg))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, g, beta, d_o, dq, dk, dv, dbeta and dg must be non-NULL");
  const void* ptrs[] = {q, k, v, g, beta, A, d_o, dht, initial_state, cu_seqlens,
                        dq, dk, dv, dbeta, dg, dh0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const Layout Lo = layout(P, true);
  if (!workspace || workspace_bytes < Lo.total)
    return fail(GDR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(Lo.total) + " bytes");
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // Recompute g_cum, A, W, U and every chunk's entry state and Vnew.  bf16
  // runs both serial passes in CP segments: the states from warmup or exact
  // segment starts, and the reverse pass the same way from segment ends
  // (exact end gradients from the reverse offsets, the transposed segment
  // transitions and a reverse scan).  fp32 runs each head whole.
  const int L = bwd_segmented(P) ? P.L : std::max(P.NTmax, 1);
  // The K = 128 bf16 gradient kernel reads A as bf16; the others as fp32.
  const bool grads_f = P.dt == gdr::DType::BF16 && P.K == 128;
  float* A_ws = grads_f ? nullptr : reinterpret_cast<float*>(ws + Lo.A);
  void* A_bf = grads_f ? static_cast<void*>(ws + Lo.A) : nullptr;
  st = run_forward_chain(P, Lo, ws, q, k, v, g, beta, scale, initial_state, cu_seqlens, nullptr,
                         nullptr, nullptr, nullptr, A_ws, A_bf, A, L, true, hs);
  if (st != GDR_OK) return st;
  if (P.NTtot == 0 && !dh0) return GDR_OK;
  const gdr::SeqTables s = tables(P, Lo, ws, L);
  hipError_t e;
  if (bwd_segmented(P)) {
    gdr::DFusedParams dp;
    dp.s = s; dp.q = q; dp.k = k; dp.Au = ws + Lo.Au; dp.d_o = d_o;
    dp.gcum = reinterpret_cast<const float*>(ws + Lo.gcum);
    dp.cert = reinterpret_cast<const float*>(ws + Lo.cert);
    dp.dht = dht; dp.dh0 = dh0; dp.dhbuf = ws + Lo.dhbuf; dp.dvn = ws + Lo.dvn;
    dp.Hq = P.Hq; dp.Hv = P.Hv; dp.seg_chunks = L; dp.warmup = P.W; dp.total_segs = P.total_segs;
    dp.log_eps = P.log_eps; dp.scale = scale;
    dp.trans = 0; dp.segtr = nullptr; dp.dhstart = nullptr; dp.hflag = nullptr;
    if (exact_cp(P, L)) {
      // the certificate decisions (reverse windows included) that the
      // forward-direction transition pass of this call recorded
      dp.hflag = reinterpret_cast<const int*>(ws + Lo.hflag);
      // reverse offsets d_s (into segtr part 1, whose b_s are spent), then
      // the exact end gradients (into hstart, whose start states are spent)
      gdr::DFusedParams tp = dp;
      tp.trans = 1;
      tp.segtr = reinterpret_cast<float*>(ws + Lo.segtr);
      if ((e = gdr::launch_dfused(P.dt, P.K, tp, P.total_segs, hs)) != hipSuccess)
        return hip_fail(e, "reverse transition launch");
      gdr::ScanParams sc;
      sc.s = s; sc.cert = dp.cert; sc.segtr = tp.segtr;
      sc.hstart = reinterpret_cast<float*>(ws + Lo.hstart);
      sc.Hv = P.Hv; sc.seg_chunks = L; sc.warmup = P.W; sc.total_segs = P.total_segs;
      sc.log_eps = P.log_eps; sc.rev = 1; sc.rev_cert = 1;
      sc.hflag = dp.hflag;
      if ((e = gdr::launch_segscan(P.K, sc, P.N * P.Hv, hs)) != hipSuccess) return hip_fail(e, "reverse scan launch");
      dp.dhstart = sc.hstart;
    }
    if ((e = gdr::launch_dfused(P.dt, P.K, dp, P.total_segs, hs)) != hipSuccess)
      return hip_fail(e, "reverse pass launch");
  } else {
    gdr::DStateParams dp;
    dp.s = s; dp.q = q; dp.k = k; dp.W = ws + Lo.W; dp.d_o = d_o;
    dp.gcum = reinterpret_cast<const float*>(ws + Lo.gcum);
    dp.dht = dht; dp.dh0 = dh0; dp.dhbuf = ws + Lo.dhbuf; dp.dvn = ws + Lo.dvn;
    dp.Hq = P.Hq; dp.Hv = P.Hv; dp.scale = scale; dp.nvb = P.nvb;
    if ((e = gdr::launch_dstate(P.dt, P.K, P.BV, dp, P.N * P.Hv * P.nvb, hs)) != hipSuccess)
      return hip_fail(e, "dstate launch");
  }
  if (P.NTtot > 0) {
    gdr::GradParams gp;
    gp.s = s; gp.q = q; gp.k = k; gp.v = v; gp.d_o = d_o; gp.hbuf = ws + Lo.hbuf;
    gp.vnew = ws + Lo.vnew; gp.dhbuf = ws + Lo.dhbuf; gp.dvn = ws + Lo.dvn;
    gp.gcum = reinterpret_cast<const float*>(ws + Lo.gcum);
    gp.beta = beta; gp.A_ws = A_ws; gp.A_bf = A_bf;
    gp.dq = dq; gp.dk = dk; gp.dv = dv; gp.dbeta = dbeta; gp.dg = dg;
    gp.Hq = P.Hq; gp.Hv = P.Hv; gp.scale = scale;
    e = grads_f ? gdr::launch_gradsf(gp, hs) : gdr::launch_grads(P.dt, P.K, gp, hs);
    if (e != hipSuccess) return hip_fail(e, "grads launch");
  }
  return GDR_OK;
}

}  // extern "C"
