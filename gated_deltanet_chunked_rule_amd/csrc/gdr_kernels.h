// gdr_kernels.h -- parameter blocks and launchers of the gfx950 kernels
// (internal to libgdr; the public C ABI is include/gdr.h).
//
// Workspace layouts (head-major so that one chunk of one head is contiguous):
//   gcum  fp32 [Hv][Ttot]          chunk-local inclusive cumsum of g
//   cert  fp32 [Hv][NTtot]         chunk gate sum, +inf if some beta|k|^2 is outside [0, 2]
//   W, U  T    [Hv][Ttot][K|V]     W = A diag(beta*Gamma) K,  U = A diag(beta) V
//   vnew  T    [Hv][Ttot][V]       Vnew = U - W h (token rows; backward only)
//   hbuf  T    [Hv][NTtot][K][V]   state entering each chunk (backward only)
//   A     fp32 [Hv][Ttot][64]      rows of the chunk's A (backward only; bf16 for K = 128)
//   dhbuf T    [Hv][NTtot][K][V]   gradient of the state leaving each chunk
//   dvn   T    [Hv][Ttot][V]       gradient of Vnew (token rows)
//   segtr fp32 [Hv][segs][2][K][V] per CP segment: M (start -> end state map) and b;
//                                  the backward then reuses part 1 for the reverse offsets d
//   hstart fp32 [Hv][segs][K][V]   exact start state of each CP segment; the backward then
//                                  reuses it for the exact state gradients at segment ends
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

enum class DType { BF16 = 0, F32 = 1 };

struct SeqTables {
  const int32_t* cu;         // [N+1] token offsets
  const int32_t* chunk_off;  // [N+1] first global chunk of each sequence
  const int32_t* seg_off;    // [N+1] first state work item of each sequence
  int N;
  long Ttot;                 // tokens in the packed batch
  int NTtot;                 // chunks (host count; device tables must agree)
  int T_uniform;             // > 0: N rows of T_uniform tokens (no cu_seqlens); the
  int segs_uniform;          //   tables are then arithmetic (segments per row) and never read
  const int32_t* seg_order;  // nullable (packed batches of unequal sequences): the state
                             //   segments by decreasing chunk steps, for the dispatch order

  __device__ __forceinline__ int nt_uniform() const { return (T_uniform + 63) / 64; }
  __device__ __forceinline__ int cu_at(int n) const { return T_uniform > 0 ? n * T_uniform : cu[n]; }
  __device__ __forceinline__ int chunk_at(int n) const { return T_uniform > 0 ? n * nt_uniform() : chunk_off[n]; }
  __device__ __forceinline__ int seg_at(int n) const { return T_uniform > 0 ? n * segs_uniform : seg_off[n]; }
  // The sequence n with off[n] <= x < off[n + 1] (the last such n among empty
  // sequences) for the chunk and segment offsets.
  __device__ __forceinline__ static int search(const int32_t* off, int N, int x) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __device__ __forceinline__ int seq_of_chunk(int c) const {
    return T_uniform > 0 ? min(c / nt_uniform(), N - 1) : search(chunk_off, N, c);
  }
  __device__ __forceinline__ int seq_of_seg(int i) const {
    return T_uniform > 0 ? min(i / segs_uniform, N - 1) : search(seg_off, N, i);
  }
};

struct PlanParams {
  const int32_t* cu_in;      // nullable: uniform rows of T tokens
  int N, T, seg_chunks;
  int32_t *cu, *chunk_off, *seg_off;
  int32_t* seg_order;        // nullable: also rank the segments by work (at most 1024 of them)
  int total_segs, warmup;
};

struct IntraParams {
  SeqTables s;
  const void *k, *v;
  const float *g, *beta;
  int Hq, Hv;
  float* gcum;
  float* g_cum_out;          // nullable, [Ttot][Hv]
  float* cert;
  void *W, *U;
  float* A_ws;               // nullable, [Hv][Ttot][64]
  void* A_bf;                // nullable, bf16 [Hv][Ttot][64] (the per-chunk gradient kernel's copy)
  void* Au;                  // non-null (bf16 forward): store A diag(beta) rows [Hv][Ttot][64]
                             //   instead of W and U (V is then not read)
  float* A_out;              // nullable, [Ttot][Hv][64]
  const float* A_in;         // nullable: use this A ([Ttot][Hv][64]) instead of inverting
};

struct StateParams {
  SeqTables s;
  const void *k, *W, *U;
  const float *gcum, *cert;
  const float* h0;           // nullable [N][Hv][K][V]
  float* ht;                 // nullable [N][Hv][K][V]
  void* hbuf;                // nullable
  void* vnew;
  int Hq, Hv;
  int seg_chunks, warmup;
  float log_eps;
  int nvb;                   // V blocks per head
};

struct FusedParams {         // forward state recurrence fused with the output
  SeqTables s;
  const void *q, *k, *W, *U;
  const void *v, *Au;        // bf16 output / transition passes: V and A diag(beta) rows instead of W, U
  const float *gcum, *cert;
  const float* h0;           // nullable [N][Hv][K][V]
  float* ht;                 // nullable [N][Hv][K][V]
  void* o;                   // [Ttot][Hv][V]
  int Hq, Hv;
  int seg_chunks, warmup, total_segs;
  float log_eps, scale;
  int trans;                 // 1: segment-transition pass (no output), 0: output pass
  float* segtr;              // transition pass: [Hv][total_segs][2][K][V] {M, b}
  const float* hstart;       // nullable: exact segment start states [Hv][total_segs][K][V]
  int rev_cert;              // 1 (backward): a head certifies only if its reverse windows do too
  int split_vnew;            // 1: bf16 output pass with Vnew as two bf16 terms (MODE 4)
  void* hbuf;                // non-null (backward recompute): store each chunk's entry state
  void* vnew;                //   and Vnew instead of the output
  int* hflag;                // nullable [N][Hv]: each head's certificate decision; the
                             //   transition pass writes it, the later passes of the call read it
};

struct DFusedParams {        // reverse state pass with CP segments (backward)
  SeqTables s;
  const void *q, *k, *Au, *d_o;   // Au: A diag(beta) rows [Hv][Ttot][64] (bf16)
  const float *gcum, *cert;
  const float* dht;          // nullable [N][Hv][K][V]
  float* dh0;                // nullable [N][Hv][K][V]
  void* dhbuf;               // [Hv][NTtot][K][V] gradient of the state leaving each chunk
  void* dvn;                 // [Hv][Ttot][V]
  int Hq, Hv;
  int seg_chunks, warmup, total_segs;
  float log_eps, scale;
  int trans;                 // 1: reverse segment offsets d_s into segtr part 1
  float* segtr;
  const float* dhstart;      // nullable: exact state gradients at the segment ends [Hv][total_segs][K][V]
  const int* hflag;          // nullable [N][Hv]: certificate decisions (reverse windows included)
                             //   of the forward-direction transition pass of the same call
};

struct ScanParams {          // exact segment start states from the segment transitions
  SeqTables s;
  const float *cert, *segtr;
  float* hstart;
  int Hv, seg_chunks, warmup, total_segs;
  float log_eps;
  int rev;                   // 1: reverse scan g_{s-1} = M_s^T g_s + d_s (state gradients)
  int rev_cert;
  const int* hflag;          // nullable [N][Hv]: certificate decisions of the transition pass
};

struct DStateParams {        // reverse state pass
  SeqTables s;
  const void *q, *k, *W, *d_o;
  const float* gcum;
  const float* dht;          // nullable
  float* dh0;                // nullable
  void* dhbuf;
  void* dvn;
  int Hq, Hv;
  float scale;
  int nvb;
};

struct GradParams {          // per-chunk gradients
  SeqTables s;
  const void *q, *k, *v, *d_o, *hbuf, *vnew, *dhbuf, *dvn;
  const float *gcum, *beta, *A_ws;
  const void* A_bf;          // bf16 copy of A (K = 128 kernel)
  void *dq, *dk, *dv;
  float *dbeta, *dg;
  int Hq, Hv;
  float scale;
};

// Kernel launchers; each returns hipGetLastError() of its launch.
hipError_t launch_plan(const PlanParams& p, hipStream_t st);
hipError_t launch_intra(DType dt, int KD, const IntraParams& p, hipStream_t st);
hipError_t launch_state(DType dt, int KD, int BV, const StateParams& p, int total_segs, bool rows,
                        hipStream_t st);
hipError_t launch_fused(DType dt, int KD, const FusedParams& p, int total_segs, hipStream_t st);
hipError_t launch_segscan(int KD, const ScanParams& p, int total_items, hipStream_t st);
hipError_t launch_dstate(DType dt, int KD, int BV, const DStateParams& p, int total_items, hipStream_t st);
hipError_t launch_dfused(DType dt, int KD, const DFusedParams& p, int total_segs, hipStream_t st);
hipError_t launch_grads(DType dt, int KD, const GradParams& p, hipStream_t st);
hipError_t launch_gradsf(const GradParams& p, hipStream_t st);   // bf16, K = V = 128, A_bf set

// Kernel timing hooks (gdr_timing.cpp).
void timing_before(const char* name, hipStream_t st);
void timing_after(hipStream_t st);

}  // namespace gdr
