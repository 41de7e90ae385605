// gdr_grads.hip -- per-chunk gradients of the chunked gated delta rule for
// K = V = 128 in bf16 on gfx950 (the other shapes use k_grads).
//
// Given the recomputed chunk states h, the state gradients dh leaving each
// chunk, Vnew and dVnew (the two serial passes of the backward), every
// (chunk, value head) is independent.  Its products, with P-like masks
// D_ts = e^{gamma_t - gamma_s} for t >= s and s the scale:
//   dPD = s D * lower(dO Vnew^T)
//   dQ  = dPD K + s diag(Gamma) dO h^T
//   dW  = -dVnew h^T,  dA = strict_lower(dW (b Gamma K)^T + dVnew (b V)^T)
//   dKb = A^T dW,  dVb = A^T dVnew,  dL = strict_lower(-A^T dA A^T)
//   dK  = dPD^T Q + (E + E^T) K + diag(b Gamma) dKb + diag(dec) Vnew dh^T,
//         E = dL * diag(b) D,  dec_t = e^{gamma_n - gamma_t}
//   dV  = diag(b) dVb,  and dbeta, dgamma from row and column sums of the
//   same terms; dg is the reverse cumulative sum of dgamma over the chunk
// (the backward listing the FlashQLA pages describe: FlashQLA curated
// summary, section "使用方式與需求").
//
// Design: a persistent grid (one 8-wave workgroup per CU) walks a contiguous
// range of (chunk, query/key head) items; each item loops over its group's
// value heads ("units") so that dq and dk are summed in registers.  Wave w
// owns feature columns 16w..16w+15 of every 64 x 128 product (h and dh rows
// 16w..16w+15 are its MFMA B operands, read once from memory straight into
// registers); 64 x 64 products are split two tiles per wave.  The token-row
// tiles (dO, Vnew, dVnew, V, Q, K) and A are copied into LDS with
// buffer-to-LDS loads; the next unit's copies are issued as soon as the
// current unit is done with each region, so the copies of one unit overlap
// the compute of the previous one.  Transposed operands come from
// transposing LDS reads; no transposed copy is stored.  Row and column sums
// go through per-wave partial arrays added in a fixed order (deterministic).
#include <math.h>

#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

template <int KD>
__global__ __launch_bounds__(FNT) void k_gradsf(GradParams p, int total_items, int per_wg) {
  using T = bf16;
  constexpr int VD = KD;
  constexpr int TE = CH * KD, TE8 = CH * CH;
  static_assert(KD == 128, "one 16-column block per wave");
  __shared__ __align__(16) T sQ[TE], sK[TE], sdO[TE], sVn[TE], sdVn[TE], sV[TE], sW[TE];
  __shared__ __align__(16) T sA2[2][TE8], sPD[TE8];
  __shared__ __align__(16) float sGc[2][CH], sBe[2][CH];
  __shared__ __align__(16) float sGam[CH], sGm[CH], sDec[CH], sBt[CH];
  __shared__ float sRowP[FNW][CH], sColP[FNW][CH], sDbP[FNW][CH], sRed[2][FNW];
  if (p.Hq < 0) {  // never taken: an ordinary store keeps the copy-only arrays from being folded away
    const T z = from_f<T>(0.f);
    sQ[threadIdx.x] = z; sK[threadIdx.x] = z; sdO[threadIdx.x] = z; sVn[threadIdx.x] = z;
    sdVn[threadIdx.x] = z; sV[threadIdx.x] = z; sA2[0][threadIdx.x] = z; sA2[1][threadIdx.x] = z;
    sGc[threadIdx.x >> 8][threadIdx.x & 63] = 0.f;
    sBe[threadIdx.x >> 8][threadIdx.x & 63] = 0.f;
  }
  // Pointers and tables are re-read from the kernel argument segment where
  // they are used (scalar loads after an opaque copy of its address; p is
  // the first argument, so it starts the segment), so the compiler does not
  // keep them in scalar registers across the unit loop, where it would
  // spill them into VGPR lanes.
  typedef const __attribute__((address_space(4))) GradParams KArgs;
  const uint64_t kargs = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  auto prm = [&]() __attribute__((always_inline)) -> KArgs* {
    uint64_t a = kargs;
    asm volatile("" : "+s"(a));
    return (KArgs*)a;
  };
  const int Hq = p.Hq, Hv = p.Hv;
  const float scale = p.scale;
  const long Ttot = p.s.Ttot;
  const int NTtot = p.s.NTtot;
  const int G = Hv / Hq;
  const int i0 = (int)blockIdx.x * per_wg;
  const int i1 = min(total_items, i0 + per_wg);
  if (i0 >= i1) return;
  const int nunits = (i1 - i0) * G;
  const int w = wave_id(), l = lane_id();
  // Lane coordinates; re-materialised opaquely at every unit so that the
  // compiler does not hoist hundreds of loop-invariant LDS addresses out of
  // the unit loop (and spill them).
  int q = l >> 4, t = l & 15;
  int dcol = 16 * w + t;                       // this wave's feature column
  // The 64 x 64 token-by-token products (dPD, dA, M1, dL) are needed on
  // their ten lower 16 x 16 tiles only.  Waves 0 and 1 take two tiles of one
  // row block, (ti, tj0) and (ti, tj0 + 1), waves 2..7 one, so that the two
  // waves of each SIMD (w and w + 4) hold 3, 3, 2 and 2 tiles:
  //   w0 (3,0) (3,1)  w1 (2,0) (2,1)  w2 (3,2)  w3 (3,3)
  //   w4 (2,2)        w5 (1,0)        w6 (1,1)  w7 (0,0)
  // Waves 2..7 also keep the six upper tiles zero where a product's
  // operand region is shared: upper tile w - 2 of M1 and of E (every unit),
  // and of the dPD / dA area (once).
  const int ti = (0x01123323 >> (4 * w)) & 15, tj0 = (0x01023200 >> (4 * w)) & 15, nt = w < 2 ? 2 : 1;
  const int zu = 4 * ((w + 6) & 7), zi = (0x211000 >> zu) & 15, zj = (0x332321 >> zu) & 15;   // upper tile w - 2 (w >= 2)

  // staged-tile element offsets: 128-wide (16 pieces a row) and 64-wide (8)
  auto t16 = [](int r, int c) __attribute__((always_inline)) { return (r * 16 + ((c >> 3) ^ stage_swz<16>(r))) * 8 + (c & 7); };
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  auto trd = [](const T* a) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
  };
  // Byte offsets of the fragment accesses.  The row swizzles use the low
  // four row bits only, and every pattern below puts the lane's coordinates
  // in those bits, so each pattern has a per-lane root offset (set at every
  // unit, see body); the step's part then adds a multiple of the row-block
  // size (16 rows of a 128-wide tile: 4096 bytes, of a 64-wide one: 2048)
  // or XORs a contraction / column block into bits 5-7, which the root's
  // piece index occupies (the piece index of a block is the XOR of the
  // block's and the lane's).  With rho = 4q + t/4:
  //   B16, B8: row 16i + t, contraction 32ks + 8q (A fragments)
  //   R16, R8: row 32ks + rho (+16), column 16m + 4(t&3) (transposing reads)
  //   V16, V8: row 16i + t, columns 16m + 4q .. +3 (8-byte reads and writes
  //            of the four columns a transposed accumulator tile holds)
  // (R16 and V16 only at this wave's column block m = w.)
  uint32_t B16, B8, R8, R16w, V8, V16w;
  auto at = [](const T* X, uint32_t off) __attribute__((always_inline)) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(X) + off);
  };
  // Fragments of V_MFMA_F32_16X16X32_BF16.  ra: row 16i + t of X, contraction
  // 32ks + 8q + j.  rb: contraction 32ks + {4q, 16 + 4q} + i over the rows of
  // X at column 16m + t (the row set of accumulator tiles 2ks, 2ks + 1).
  // rt: contraction 32ks + 8q + j over the rows of X at column c0 + t.
  auto ra16 = [&](const T* X, int i, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(at(X, 4096 * i + (B16 ^ (64 * ks))));
  };
  auto ra8 = [&](const T* X, int i, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(at(X, 2048 * i + (B8 ^ (64 * ks))));
  };
  auto rb16w = [&](const T* X, int ks) __attribute__((always_inline)) {   // m = w
    const T* a = at(X, 8192 * ks + R16w);
    return cat4(trd(a), trd(a + 2048));
  };
  auto rb8 = [&](const T* X, int ks, int m) __attribute__((always_inline)) {
    const T* a = at(X, 4096 * ks + (R8 ^ (32 * m)));
    return cat4(trd(a), trd(a + 1024));
  };
  auto rt16 = [&](const T* X, int ks, int c0) __attribute__((always_inline)) {
    const int r = 32 * ks + 8 * q + (t >> 2), c = c0 + 4 * (t & 3);
    return cat4(trd(X + t16(r, c)), trd(X + t16(r + 4, c)));
  };
  // Every product below is computed with its operands swapped (the A and B
  // fragments have the same register layout), so that an accumulator tile
  // holds the transposed block: lane (q, t) has row 16i + t and the four
  // columns 16m + 4q + e, e < 4, which leave as one 8-byte store.
  // X[16i + t][16w + 4q + e] of a 128-wide tile, as floats
  auto row4 = [&](const T* X, int i) __attribute__((always_inline)) {
    const uint2 u = *reinterpret_cast<const uint2*>(at(X, 4096 * i + V16w));
    f32x4 f;
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    return f;
  };
  // F[16i + 4q + e], e < 4 (per-token factors at a tile's columns)
  auto fac4 = [&](const float* F, int i) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(F + 16 * i + 4 * q);
  };
  // a transposed accumulator tile (row block i, column block m) into a 64 x 64 LDS matrix
  auto st_t8 = [&](T* X, int i, int m, f32x4 v) __attribute__((always_inline)) {
    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(X) + 2048 * i + (V8 ^ (32 * m))) = pack4_bf16(v);
  };
  auto mf = [](bf16x8 a, bf16x8 b, f32x4 c) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  };

  // per-lane byte offsets of the tile copies (rows past the chunk read as 0)
  uint32_t off_qk[2], off_hv[2], off_ws[2], off_a[1];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pidx = 64 * (w + FNW * j) + l;
    const int r = pidx >> 4, c = (pidx & 15) ^ stage_swz<16>(r);
    off_qk[j] = (uint32_t)(r * Hq * KD * 2 + c * 16);
    off_hv[j] = (uint32_t)(r * Hv * VD * 2 + c * 16);
    off_ws[j] = (uint32_t)(r * VD * 2 + c * 16);
  }
  {
    const int pidx = 64 * w + l;
    const int r = pidx >> 3, c = (pidx & 7) ^ stage_swz<8>(r);
    off_a[0] = (uint32_t)(r * CH * 2 + c * 16);
  }
  // Units in order: value head gi of q/k head hk of chunk c, items
  // (chunk, q/k head) i0 .. i1 - 1, the next unit derived from the current.
  struct Unit { int c, hk, h, gi, t0, len; };
  int cc = -1, ct0 = 0, clen = 0;   // the last chunk looked up (the chunk changes every Hq items)
  auto locate = [&](Unit& u) __attribute__((always_inline)) -> bool {
    u.h = u.hk * G + u.gi;
    if (u.c != cc) {
      KArgs* pa = prm();
      SeqTables st;
      st.cu = pa->s.cu;
      st.chunk_off = pa->s.chunk_off;
      st.seg_off = pa->s.seg_off;
      st.N = pa->s.N;
      st.Ttot = pa->s.Ttot;
      st.NTtot = pa->s.NTtot;
      st.T_uniform = pa->s.T_uniform;
      st.segs_uniform = pa->s.segs_uniform;
      st.seg_order = pa->s.seg_order;
      int n;
      if (!locate_chunk_b(st, u.c, n, ct0, clen)) return false;
      cc = u.c;
    }
    u.t0 = ct0;
    u.len = clen;
    return true;
  };
  auto advance = [&](const Unit& a, Unit& u) __attribute__((always_inline)) {
    u = a;
    if (++u.gi == G) {
      u.gi = 0;
      if (++u.hk == Hq) { u.hk = 0; ++u.c; }
    }
  };
  int wsc = w;   // the wave id in a scalar register, made opaque at every unit (see body)
  // (nt: tiles that only this unit reads; q and k serve the group's value heads)
  auto tile = [&](T* dst, const void* base, long elem0, long row_elems, int len, const uint32_t* off, auto ntc)
      __attribute__((always_inline)) {
    lds_copy_tile<2, 16, FNW, 8, decltype(ntc)::value != 0>(dst, rsrc_words((const T*)base + elem0, (long)len * row_elems * 2), off, wsc);
  };
  auto copy_dO_Vn = [&](const Unit& u) __attribute__((always_inline)) {
    KArgs* pa = prm();
    tile(sdO, pa->d_o, ((long)u.t0 * Hv + u.h) * VD, (long)Hv * VD, u.len, off_hv, ic<1>());
    tile(sVn, pa->vnew, ((long)u.h * Ttot + u.t0) * VD, VD, u.len, off_ws, ic<1>());
  };
  auto copy_Q = [&](const Unit& u) __attribute__((always_inline)) {
    tile(sQ, prm()->q, ((long)u.t0 * Hq + u.hk) * KD, (long)Hq * KD, u.len, off_qk, ic<0>());
  };
  auto copy_K = [&](const Unit& u) __attribute__((always_inline)) {
    tile(sK, prm()->k, ((long)u.t0 * Hq + u.hk) * KD, (long)Hq * KD, u.len, off_qk, ic<0>());
  };
  auto copy_dVn_V = [&](const Unit& u) __attribute__((always_inline)) {
    KArgs* pa = prm();
    tile(sdVn, pa->dvn, ((long)u.h * Ttot + u.t0) * VD, VD, u.len, off_ws, ic<1>());
    tile(sV, pa->v, ((long)u.t0 * Hv + u.h) * VD, (long)Hv * VD, u.len, off_hv, ic<1>());
  };
  auto copy_A_gates = [&](const Unit& u, auto abc) __attribute__((always_inline)) {   // into buffer ab
    constexpr int ab = decltype(abc)::value;
    KArgs* pa = prm();
    lds_copy_tile<1, 8, FNW, 8, true>(&sA2[ab][0],
                                rsrc_words((const T*)pa->A_bf + ((long)u.h * Ttot + u.t0) * CH, (long)u.len * CH * 2),
                                off_a, wsc);
    if (w == 0) {
      const i32x4v gr = rsrc_words(pa->gcum + (long)u.h * Ttot + u.t0, (long)u.len * 4);
      lds_copy4(gr, (uint32_t)l * 4u, lds_addr(&sGc[ab][0]));
      const i32x4v br = rsrc_words(pa->beta + (long)u.t0 * Hv + u.h, ((long)(u.len - 1) * Hv + 1) * 4);
      lds_copy4(br, (uint32_t)(l * Hv * 4), lds_addr(&sBe[ab][0]));
    }
  };
  // rows 16w..16w+15 of h and dh as B fragments (contraction over V)
  auto load_hd = [&](const Unit& u, bf16x8 (&hf)[4], bf16x8 (&df)[4]) __attribute__((always_inline)) {
    const long base = (((long)u.h * NTtot + u.c) * KD + dcol) * VD + 8 * q;
    KArgs* pa = prm();
    const T* hb = (const T*)pa->hbuf + base;
    const T* db = (const T*)pa->dhbuf + base;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      hf[ks] = *reinterpret_cast<const bf16x8*>(hb + 32 * ks);
      df[ks] = *reinterpret_cast<const bf16x8*>(db + 32 * ks);
    }
  };

  Unit cu;
  cu.c = i0 / Hq;
  cu.hk = i0 - cu.c * Hq;
  cu.gi = 0;
  if (!locate(cu)) return;
  copy_Q(cu);
  copy_K(cu);
  copy_dO_Vn(cu);
  copy_dVn_V(cu);
  copy_A_gates(cu, ic<0>());
  if (w >= 2) {
    const int r = 16 * zi + t, c = 16 * zj + 4 * q;
    *reinterpret_cast<uint2*>(sPD + (r * 8 + ((c >> 3) ^ stage_swz<8>(r))) * 8 + (c & 7)) = make_uint2(0u, 0u);
  }
  // the first unit's copies have landed (later units wait at the end of the previous one)
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  f32x4 dq[4], dk[4];
  // raw Q K^T and K K^T tiles of this wave, transposed like the products
  // they scale; they depend on q and k only, so they are formed at the
  // first unit of an item and kept for its other value heads
  f32x4 Sqk[2], Skk[2];
  bf16x8 kt1[2], kt2[2];   // K fragments at column block w: rt (for dPD K, E K) and rb (for E^T K)

  // One unit with its A and gate buffers ab (a compile-time index: the loop
  // is unrolled by two); false when there is no next unit.
  auto body = [&](auto abc, int j) __attribute__((always_inline)) -> bool {
    constexpr int ab = decltype(abc)::value;
    asm volatile("" : "+v"(q), "+v"(t), "+v"(dcol));
    {
      const int rho = 4 * q + (t >> 2);
      B16 = 256 * t + 16 * (q ^ stage_swz<16>(t));
      B8 = 128 * t + 16 * (q ^ stage_swz<8>(t));
      R8 = 128 * rho + 8 * (t & 1) + 16 * (((t >> 1) & 1) ^ stage_swz<8>(rho));
      R16w = (256 * rho + 8 * (t & 1) + 16 * (((t >> 1) & 1) ^ stage_swz<16>(rho))) ^ (32 * w);
      V8 = 128 * t + 16 * ((q >> 1) ^ stage_swz<8>(t)) + 8 * (q & 1);
      V16w = (256 * t + 16 * ((q >> 1) ^ stage_swz<16>(t)) + 8 * (q & 1)) ^ (32 * w);
    }
    wsc = w;
    asm volatile("" : "+s"(wsc));
    Unit nu;
    advance(cu, nu);
    const bool has_next = j + 1 < nunits && locate(nu);
    const bool new_item = cu.gi == 0;
    const bool next_new = has_next && nu.gi == 0;
    const T* sA = &sA2[ab][0];
    const float* gcb = &sGc[ab][0];
    const float* beb = &sBe[ab][0];
    const int len = cu.len, t0 = cu.t0, h = cu.h;
    // this unit's h and dh fragments: issued first, needed after the dPD tiles
    bf16x8 Hf[4], Df[4];
    load_hd(cu, Hf, Df);

    // ---- unit start: this unit's copies have landed (waited at the end of
    // the previous unit); gate factors and zeroed per-wave partial sums.
    // Every wave writes the same factor values, so each wave reads what it
    // wrote itself and no barrier is needed here: the previous unit's final
    // barrier already keeps these writes after every read of the old values.
    {
      const float gl = gcb[len - 1], gv = gcb[l];
      const float gam = l < len ? gv : gl;
      sGam[l] = gam;
      sGm[l] = l < len ? __expf(gam) : 0.f;
      sDec[l] = l < len ? __expf(gl - gam) : 0.f;
      sBt[l] = l < len ? beb[l] : 0.f;
    }
    sRowP[w][l] = 0.f;
    sColP[w][l] = 0.f;
    sDbP[w][l] = 0.f;
    if (new_item) {   // cached K fragments, zero dq and dk
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kt1[ks] = rt16(sK, ks, 16 * w);
        kt2[ks] = rb16w(sK, ks);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) { dq[tt] = zero4(); dk[tt] = zero4(); }
    }

    // ---- phase 1: dPD tiles; dO h^T, dVnew h^T, Vnew dh^T (column split)
    {
      // dO Vnew^T, transposed tiles: row 16ti + t, columns 16(tj0 + m) + 4q + e
      if (new_item) {
        Sqk[0] = zero4();
        Sqk[1] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 aq = ra16(sQ, ti, ks);
#pragma unroll
          for (int m = 0; m < 2; ++m)
            if (m < nt) Sqk[m] = mf(ra16(sK, tj0 + m, ks), aq, Sqk[m]);
        }
      }
      f32x4 dP[2] = {zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = ra16(sdO, ti, ks);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (m < nt) dP[m] = mf(ra16(sVn, tj0 + m, ks), a, dP[m]);
      }
      const int r = 16 * ti + t;
      const float gr = sGam[r];
      float rx = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m >= nt) break;
        const f32x4 gc = fac4(sGam, tj0 + m);
        float cx[4];
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * (tj0 + m) + 4 * q + e;
          const float v = (r >= c && r < len) ? scale * __expf(gr - gc[e]) * dP[m][e] : 0.f;
          const float x = v * Sqk[m][e];
          rx += x;
          cx[e] = x;
          pv[e] = v;
        }
        st_t8(sPD, ti, tj0 + m, pv);
        const float cs = row16_sums4(cx);   // column 16(tj0 + m) + 4q + t/4
        if ((t & 3) == 0) sColP[w][16 * (tj0 + m) + 4 * q + (t >> 2)] -= cs;
      }
      rx = col_group_sum(rx);
      if (q == 0) sRowP[w][r] += rx;
    }
    // Three passes over h and dh (rows 16w..16w+15 as B fragments), each
    // folded right away: s Gamma_t dO h^T into dq, -dVnew h^T (dW) into LDS
    // rows, dec_t Vnew dh^T into dk; with the row sums they feed.  Rows of
    // the 64 x 16 blocks below are tokens 16i + t, columns 16w + 4q + e.
    {  // dVb = A^T dVnew (needs neither h nor dh): dv and its dbeta terms
      f32x4 vb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) vb[st] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 bd = rb16w(sdVn, ks);
#pragma unroll
        for (int st = 0; st < 4; ++st) vb[st] = mf(bd, rb8(sA, ks, st), vb[st]);
      }
      // dv rows through a descriptor covering the chunk's rows (rows past
      // the chunk are dropped by the range check)
      const rsrc_t dvr = make_rsrc_u((const T*)prm()->dv + ((long)t0 * Hv + h) * VD, (long)len * Hv * VD * 2);
      const uint32_t dvo = (uint32_t)((t * Hv * VD + 16 * w + 4 * q) * 2);
      float dbL[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float bt = sBt[16 * st + t];
        const f32x4 ve = row4(sV, st);
        float db = 0.f;
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          db += vb[st][e] * ve[e];
          o[e] = bt * vb[st][e];
        }
        dbL[st] = db;
        buf_store8(dvr, dvo + (uint32_t)(16 * st * Hv * VD * 2), pack4_bf16(o));
      }
      sDbP[w][16 * q + t] += group_sums4(dbL);
    }
    float hdp = 0.f, rsum = 0.f;
    float rowL[4] = {0.f, 0.f, 0.f, 0.f};   // per-lane row partials (rows 16tt + t)
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const T* X = pass == 0 ? sdO : pass == 1 ? sdVn : sVn;
      f32x4 acc[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 b = pass == 2 ? Df[ks] : Hf[ks];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[tt] = mf(b, ra16(X, tt, ks), acc[tt]);
        if (pass == 2) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          struct Pairs { bf16x2 v[4]; };
          const Pairs hp = __builtin_bit_cast(Pairs, Hf[ks]), dp = __builtin_bit_cast(Pairs, Df[ks]);
#pragma unroll
          for (int i = 0; i < 4; ++i) hdp = __builtin_amdgcn_fdot2_f32_bf16(hp.v[i], dp.v[i], hdp, false);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (pass == 0) {
          const float gm = sGm[16 * tt + t];
          const f32x4 qe = row4(sQ, tt);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float vq = scale * gm * acc[tt][e];   // s Gamma_t (dO h^T)
            dq[tt][e] += vq;
            rowL[tt] += vq * qe[e];
          }
        } else if (pass == 1) {   // dW rows
          *reinterpret_cast<uint2*>(reinterpret_cast<char*>(sW) + 4096 * tt + V16w) = pack4_bf16(-acc[tt]);
        } else {
          const float dc = sDec[16 * tt + t];
          const f32x4 ke = row4(sK, tt);
          float rk = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float vk = dc * acc[tt][e];             // dec_t (Vnew dh^T)
            dk[tt][e] += vk;
            rk += vk * ke[e];
          }
          rsum += rk;
          rowL[tt] -= rk;
        }
      }
    }
    sRowP[w][16 * q + t] += group_sums4(rowL);
    rsum = wave_sum(rsum);
    hdp = wave_sum(hdp);
    if (l == 0) { sRed[0][w] = rsum; sRed[1][w] = hdp; }
    lds_barrier();   // dPD and dW rows complete; dO and Vnew are no longer read
    if (has_next) {
      copy_dO_Vn(nu);
      copy_A_gates(nu, ic<1 - ab>());
    }
    {  // dQ += dPD K;  dK += dPD^T Q
      bf16x8 bq[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bq[ks] = rb16w(sQ, ks);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dq[tt] = mf(kt1[ks], ra8(sPD, tt, ks), dq[tt]);
          dk[tt] = mf(bq[ks], rb8(sPD, ks, tt), dk[tt]);
        }
    }
    lds_barrier();   // Q and dPD are no longer read
    if (next_new) copy_Q(nu);

    // ---- phase 2: dA tiles; dKb = A^T dW and dVb = A^T dVnew (column split)
    T* sdA = sPD;
    {
      if (new_item) {
        Skk[0] = zero4();
        Skk[1] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 ak = ra16(sK, ti, ks);
#pragma unroll
          for (int m = 0; m < 2; ++m)
            if (m < nt) Skk[m] = mf(ra16(sK, tj0 + m, ks), ak, Skk[m]);
        }
      }
      f32x4 ta[2] = {zero4(), zero4()}, tb[2] = {zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a1 = ra16(sW, ti, ks), a2 = ra16(sdVn, ti, ks);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (m < nt) {
            ta[m] = mf(ra16(sK, tj0 + m, ks), a1, ta[m]);
            tb[m] = mf(ra16(sV, tj0 + m, ks), a2, tb[m]);
          }
      }
      const int r = 16 * ti + t;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m >= nt) break;
        const f32x4 btc = fac4(sBt, tj0 + m), gmc = fac4(sGm, tj0 + m);
        f32x4 av;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * (tj0 + m) + 4 * q + e;
          av[e] = (r > c) ? btc[e] * (gmc[e] * ta[m][e] + tb[m][e]) : 0.f;
        }
        st_t8(sdA, ti, tj0 + m, av);
      }
    }
    {  // dKb = A^T dW, rows s of A^T in blocks st
      f32x4 kb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) kb[st] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 bw = rb16w(sW, ks);
#pragma unroll
        for (int st = 0; st < 4; ++st) kb[st] = mf(bw, rb8(sA, ks, st), kb[st]);
      }
      float rowK[4], dbL[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float gm = sGm[16 * st + t], bg = sBt[16 * st + t] * gm;
        const f32x4 ke = row4(sK, st);
        float kk = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[st][e] += bg * kb[st][e];
          kk += kb[st][e] * ke[e];
        }
        rowK[st] = bg * kk;
        dbL[st] = gm * kk;
      }
      sRowP[w][16 * q + t] += group_sums4(rowK);
      sDbP[w][16 * q + t] += group_sums4(dbL);
    }
    lds_barrier();   // dA complete; dW, dVnew, V and K are no longer read from LDS
    if (has_next) {
      copy_dVn_V(nu);
      if (next_new) copy_K(nu);
    }

    // ---- phase 3: M1 = A^T dA; dL = -M1 A^T -> E; dK += E K + E^T K
    T* sM1 = sW;
    T* sE = sW + TE8;
    {
      f32x4 m1[2] = {zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = rb8(sA, ks, ti);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (m < nt) m1[m] = mf(rb8(sdA, ks, tj0 + m), a, m1[m]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (m < nt) st_t8(sM1, ti, tj0 + m, m1[m]);
      if (w >= 2) {   // upper tiles of M1 and E: the dW rows were there
        st_t8(sM1, zi, zj, zero4());
        st_t8(sE, zi, zj, zero4());
      }
    }
    lds_barrier();
    {
      f32x4 dl[2] = {zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = ra8(sM1, ti, ks);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (m < nt) dl[m] = mf(ra8(sA, tj0 + m, ks), a, dl[m]);
      }
      const int r = 16 * ti + t;
      const float gr = sGam[r], btr = sBt[r];
      float rx = 0.f, bs = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m >= nt) break;
        const f32x4 gc = fac4(sGam, tj0 + m);
        float cx[4];
        f32x4 evv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * (tj0 + m) + 4 * q + e;
          float ev = 0.f, x = 0.f;
          if (r > c) {
            const float D = __expf(gr - gc[e]);
            const float dlv = -dl[m][e];
            const float y = dlv * D * Skk[m][e];
            bs += y;
            ev = dlv * btr * D;
            x = btr * y;
            rx += x;
          }
          cx[e] = x;
          evv[e] = ev;
        }
        st_t8(sE, ti, tj0 + m, evv);
        const float cs = row16_sums4(cx);   // column 16(tj0 + m) + 4q + t/4
        if ((t & 3) == 0) sColP[w][16 * (tj0 + m) + 4 * q + (t >> 2)] -= cs;
      }
      rx = col_group_sum(rx);
      bs = col_group_sum(bs);
      if (q == 0) {
        sRowP[w][r] += rx;
        sDbP[w][r] += bs;
      }
    }
    lds_barrier();   // E complete; every partial sum is in
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dk[tt] = mf(kt1[ks], ra8(sE, tt, ks), dk[tt]);
        dk[tt] = mf(kt2[ks], rb8(sE, ks, tt), dk[tt]);
      }
    // dgamma row sums and dg as their reverse cumulative sum on wave 3,
    // dbeta on wave 2 (both on the SIMDs with fewer 64 x 64 tiles)
    if (w == 3) {
      float dgm = 0.f;
#pragma unroll
      for (int ww = 0; ww < FNW; ++ww) dgm += sRowP[ww][l] + sColP[ww][l];
      if (l == len - 1) {
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int ww = 0; ww < FNW; ++ww) { r0 += sRed[0][ww]; r1 += sRed[1][ww]; }
        dgm += r0 + __expf(sGam[CH - 1]) * r1;
      }
      dgm = (l < len) ? dgm : 0.f;
      const float rev = __shfl(dgm, 63 - l, 64);
      const float sc = wave_inclusive_scan(rev);
      const float dgv = __shfl(sc, 63 - l, 64);
      if (l < len) prm()->dg[(long)(t0 + l) * Hv + h] = dgv;
    } else if (w == 2) {
      float db = 0.f;
#pragma unroll
      for (int ww = 0; ww < FNW; ++ww) db += sDbP[ww][l];
      if (l < len) prm()->dbeta[(long)(t0 + l) * Hv + h] = db;
    }
    if (cu.gi == G - 1) {   // the group's dq and dk rows
      KArgs* pa = prm();
      const long e0 = ((long)t0 * Hq + cu.hk) * KD, nb = (long)len * Hq * KD * 2;
      const rsrc_t dqr = make_rsrc_u((const T*)pa->dq + e0, nb), dkr = make_rsrc_u((const T*)pa->dk + e0, nb);
      const uint32_t o = (uint32_t)((t * Hq * KD + 16 * w + 4 * q) * 2);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {   // row 16tt + t (rows past the chunk are dropped)
        const uint32_t ot = o + (uint32_t)(16 * tt * Hq * KD * 2);
        buf_store8(dqr, ot, pack4_bf16(dq[tt]));
        buf_store8(dkr, ot, pack4_bf16(dk[tt]));
      }
    }
    // the next unit's copies have landed; every wave is done with this unit
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (!has_next) return false;
    cu = nu;
    return true;
  };
  for (int j = 0; j < nunits; j += 2) {
    if (!body(ic<0>(), j) || !body(ic<1>(), j + 1)) break;
  }
}

hipError_t launch_gradsf(const GradParams& p, hipStream_t st) {
  const int total = p.s.NTtot * p.Hq;
  if (total <= 0) return hipSuccess;
  const int nwg = std::min(total, 256);
  const int per_wg = (total + nwg - 1) / nwg;
  timing_before("chunk_grads", st);
  hipLaunchKernelGGL((k_gradsf<128>), dim3(nwg), dim3(FNT), 0, st, p, total, per_wg);
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

}  // namespace gdr
