// The whole MoE layer in one persistent launch ("PagedWeight", §3.3: routing,
// expert activation, down projection and output accumulation in one fused
// kernel that reads the weight pages at each block's committed bitwidth).
//
// The work is a sequence of units, in this order: [bf16 -> fp16 conversion, one per token]
// [router logits] [top-K] [grouping, one per group] [gate_up, one per (item,
// 128-column tile)] [down, one per (item, 128-row tile)] [combine]. Each
// workgroup repeatedly takes the next unit from a global counter and runs it;
// a unit first waits until the units it reads from have completed (counters
// released at agent scope after the producer's writes, acquired before the
// consumer's reads). A unit only waits on units earlier in the sequence, and
// those were taken by workgroups that are running and wait only on still
// earlier units, so the earliest unfinished unit can always proceed: no
// assumption about how many workgroups are resident is needed. A down unit
// waits only for the gate_up units of its own group, so down work starts while
// other groups' gate_up units are still running.
//
// Counters (256 bytes apart) live at the start of the workspace. They must be zero when
// the launch starts; the last workgroup to finish sets them back to zero, so a
// workspace stays ready for the next launch (including graph replays). Every
// wait is bounded: a wait that runs out (which correct use never causes) sets
// an error word, the remaining units skip their work, and the output is NaN.
#include "k_ffn_body.h"
#include "k_route_body.h"

namespace mpb {

namespace {

constexpr int kMaxGroupsF = 512 + 64;
constexpr uint32_t kSpinLimit = 1u << 20;  // polls before a wait gives up (~2 s at the longest sleep)
constexpr int kCtrStride = 64;             // counters 256 bytes apart: polls spread over memory channels

enum : int {
  C_HEAD = 0,   // next unit
  C_EXIT = 1,   // workgroups finished
  C_CONV = 2,   // conversion units done
  C_LOGIT = 3,  // logits units done
  C_TOPK = 4,   // top-K units done
  C_GROUP = 5,  // grouping units done
  C_DOWN = 6,   // down units done (with work)
  C_ERR = 7,    // a wait ran out
  C_GU = 8      // [NB] gate_up units done per group
};

}  // namespace

struct FusedParams {
  FfnParams f;          // FFN view; f.topk_idx / f.topk_w alias idx_out / w_out
  const uint16_t* x;    // activations as given (fp16 or bf16 bits)
  const float* W;       // router weights [E][H]
  const float* bias;    // [E] or null
  double* logits;       // [T][E]
  int32_t* idx_out;     // [T][K]
  float* w_out;         // [T][K]
  uint32_t* ctr;        // counters (see above)
  int qmax;
  uint32_t slot_off;    // LDS byte offset of the unit slot and the wait flag
  int n_conv, n_logit, n_topk, n_group, n_gu, n_dn, n_comb;
  int ntile_gu, ntile_dn;
  int logit_mfma;       // logits on the fp64 matrix cores (16 x 16 tiles), as the per-phase router does
  int ks;               // hidden parts of the vector-path logits (route_ksplit)
};

namespace {

__device__ __forceinline__ uint32_t* ctr(const FusedParams& P, int c) { return P.ctr + c * kCtrStride; }

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (whole workgroup) until counter c reaches target; returns false if the
// workspace is in the error state (a wait ran out here or earlier). Data that
// units hand to each other is read and written with device-coherent accesses
// (ld_co / st_co), so observing the counter is all a consumer needs: no cache
// invalidation.
__device__ __forceinline__ bool wait_count(const FusedParams& P, int c, uint32_t target, uint32_t* flag) {
  if (threadIdx.x == 0) {
    // polls back off from ~64 to ~4096 cycles apart, so waiting workgroups
    // add little memory traffic; the error word is checked every 16 polls
    uint32_t n = 0;
    int nap = 0;
    while (ld_relaxed(ctr(P, c)) < target) {
      if (nap == 0) __builtin_amdgcn_s_sleep(1);
      else if (nap == 1) __builtin_amdgcn_s_sleep(4);
      else if (nap == 2) __builtin_amdgcn_s_sleep(16);
      else __builtin_amdgcn_s_sleep(64);
      nap += nap < 3;
      if ((++n & 15) == 0 && ld_relaxed(ctr(P, C_ERR)) != 0) break;
      if (n >= kSpinLimit) {
        __hip_atomic_store(ctr(P, C_ERR), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    *flag = ld_relaxed(ctr(P, C_ERR));
  }
  __syncthreads();
  const bool ok = *flag == 0;
  __syncthreads();  // every thread has read the flag before thread 0 may rewrite it
  return ok;
}

// Count the unit as done once every wave's device-coherent stores have
// completed (stores are counted in vmcnt): they are then in memory, where a
// consumer that sees the counter will read them.
__device__ __forceinline__ void mark_done(uint32_t* c) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads the work item of a gate_up (list 0) or down (list 1) unit once, in
// thread 0, and hands it to the workgroup through LDS (slot[2..4]), so every
// wave takes the same branches: returns false for a unit past the list.
__device__ __forceinline__ bool unit_item(const FfnParams& p, int list, int item, uint32_t* slot, int& e, int& t0,
                                          int& nt, int& cnt_e) {
  if (threadIdx.x == 0) {
    const int n = ld_co<true>(p.n_items + list);
    slot[2] = item < n ? 1u : 0u;
    if (item < n) {
      const int v = ld_co<true>((list ? p.items_dn : p.items) + item);
      slot[3] = (uint32_t)v;
      slot[4] = (uint32_t)ld_co<true>(p.counts + (v >> 16));
    }
  }
  __syncthreads();
  const bool live = slot[2] != 0;
  const int v = (int)slot[3];
  cnt_e = (int)slot[4];
  __syncthreads();
  if (!live) return false;
  const int tpi = list ? p.tpi_dn : p.tpi;
  e = v >> 16;
  t0 = (v & 0xffff) * tpi;
  nt = min(cnt_e - t0, tpi);
  return true;
}

// Grouping of group e with 512 threads (the same result as the per-phase
// grouping kernel): histogram of the routed ids in LDS, this group's offset,
// its positions in both bitwidth-ordered item lists and the item totals, then
// a ballot-ordered stable scatter of its entries.
__device__ __forceinline__ void group_unit(const FfnParams& p, int e, int* sm, int tid) {
  int* hist = sm;                          // [kMaxGroupsF]
  int* red = sm + kMaxGroupsF;             // [5][8]
  int* wtot = red + 40;                    // [8]
  const int lane = tid & 63, w = tid >> 6;
  const int T = p.T, K = p.K, S = p.S, E = p.E, KS = K + S, TK = T * K;
  for (int i = tid; i < E; i += 512) hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < TK; j += 512) {
    const int x = ld_co<true>(p.topk_idx + j);
    if (x >= 0 && x < E) atomicAdd(&hist[x], 1);
  }
  __syncthreads();
  const int qg = p.q[2 * e], qd = p.q[2 * e + 1];
  const int mine = e < E ? hist[e] : T;
  const int ni = (mine + p.tpi - 1) / p.tpi, ni_dn = (mine + p.tpi_dn - 1) / p.tpi_dn;
  int a[5] = {0, 0, 0, 0, 0};
  for (int j = tid; j < p.NB; j += 512) {
    const int cnt = j < E ? hist[j] : T;
    const int n = (cnt + p.tpi - 1) / p.tpi, n_dn = (cnt + p.tpi_dn - 1) / p.tpi_dn;
    const int qjg = p.q[2 * j], qjd = p.q[2 * j + 1];
    if (j < e) a[0] += cnt;
    if (qjg > qg || (qjg == qg && j < e)) a[1] += n;
    if (qjd > qd || (qjd == qd && j < e)) a[2] += n_dn;
    a[3] += n;
    a[4] += n_dn;
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a[i] += __shfl_xor(a[i], o);
    if (lane == 0) red[i * 8 + w] = a[i];
  }
  __syncthreads();
  int r[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    r[i] = 0;
#pragma unroll
    for (int v = 0; v < 8; ++v) r[i] += red[i * 8 + v];
  }
  const int off = r[0], igu = r[1], idn = r[2];
  if (tid == 0) {
    st_co<true>(p.offsets + e, off);
    st_co<true>(p.counts + e, mine);
    if (e == p.NB - 1) st_co<true>(p.offsets + p.NB, off + mine);
    if (e == 0) {
      st_co<true>(p.n_items, r[3]);
      st_co<true>(p.n_items + 1, r[4]);
    }
  }
  for (int sp = tid; sp < ni; sp += 512) st_co<true>(p.items + igu + sp, (e << 16) | sp);
  for (int sp = tid; sp < ni_dn; sp += 512) st_co<true>(p.items_dn + idn + sp, (e << 16) | sp);
  if (e < E) {
    int run = 0;
    for (int b0 = 0; b0 < TK; b0 += 512) {
      const int j = b0 + tid;
      const int x = j < TK ? ld_co<true>(p.topk_idx + j) : -1;
      const bool m = x == e;
      const unsigned long long bal = __ballot(m);
      const int lp = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int wp = 0, tot = 0;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        wp += v < w ? wtot[v] : 0;
        tot += wtot[v];
      }
      if (m) {
        const int pos = off + run + wp + lp;
        const int t = j / K, k = j - t * K;
        st_co<true>(p.ptok + pos, t);
        st_co<true>(p.pw + pos, ld_co<true>(p.topk_w + j));
        st_co<true>(p.ent + pos, t * KS + k);
      }
      run += tot;
      __syncthreads();
    }
  } else {
    const int s = e - E;
    for (int t = tid; t < T; t += 512) {
      const int pos = off + t;
      st_co<true>(p.ptok + pos, t);
      st_co<true>(p.pw + pos, 1.0f);
      st_co<true>(p.ent + pos, t * KS + K + s);
    }
  }
}

__device__ __forceinline__ void gate_up_unit(const FusedParams& P, int u, uint16_t* lds, uint32_t* slot, int tid) {
  const FfnParams& p = P.f;
  const int item = u / P.ntile_gu, it = u - item * P.ntile_gu;
  int e, t0, nt, cnt;
  if (!unit_item(p, 0, item, slot, e, t0, nt, cnt)) return;
  ItemRow wi;
  item_fields<true>(p, 2 * e, e, t0, p.tpi, wi);
  wi.nt = nt;
  const int q = wi.q;
  const uint32_t lut_bytes = 256u << P.qmax;
  switch (q < 3 || q > P.qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3:  // pair tables (the launch holds their LDS, fused_lds_bytes)
      if (nt <= kDbTok) gate_up_body<3, 1, true, true, true, true>(p, wi, it, lds, kPairTableBytes, tid);
      else gate_up_body<3, 1, true, true, false, true>(p, wi, it, lds, kPairTableBytes, tid);
      break;
    case 4:
      if (nt <= kDbTok) gate_up_body<4, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid);
      else gate_up_body<4, 1, true>(p, wi, it, lds, lut_bytes, tid);
      break;
    case 5:
      if (nt <= kDbTok) gate_up_body<5, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid);
      else gate_up_body<5, 1, true>(p, wi, it, lds, lut_bytes, tid);
      break;
    case 6:
      if (nt <= kDbTok) gate_up_body<6, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid);
      else gate_up_body<6, 1, true>(p, wi, it, lds, lut_bytes, tid);
      break;
    case 7:
      if (nt <= kDbTok) gate_up_body<7, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid);
      else gate_up_body<7, 1, true>(p, wi, it, lds, lut_bytes, tid);
      break;
    case 8:
      if (nt <= kDbTok) gate_up_body<8, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid);
      else gate_up_body<8, 1, true>(p, wi, it, lds, lut_bytes, tid);
      break;
    default: {
      const size_t o = (size_t)wi.base * p.I + it * 64;
      for (int i = tid; i < nt * 64; i += kThreads) {
        p.hhi[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0x7e00;  // fp16 NaN
        p.hlo[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0;
      }
    }
  }
  mark_done(ctr(P, C_GU + e));
}

__device__ __forceinline__ void down_unit(const FusedParams& P, int u, uint16_t* lds, uint32_t* slot, int tid) {
  const FfnParams& p = P.f;
  // unit u: K range u % dn_split of tile (u / dn_split) % ntile_dn of item (u / dn_split) / ntile_dn
  const int b = u / p.dn_split, ksi = u - b * p.dn_split;
  const int item = b / P.ntile_dn, it = b - item * P.ntile_dn;
  int e, t0, nt, cnt;
  if (!unit_item(p, 1, item, slot, e, t0, nt, cnt)) return;
  uint32_t* flag = slot + 1;
  // h of group e is complete once all of its gate_up units are
  const uint32_t need = (uint32_t)((cnt + p.tpi - 1) / p.tpi) * P.ntile_gu;
  if (!wait_count(P, C_GU + e, need, flag)) return;
  ItemRow wi;
  item_fields<true>(p, 2 * e + 1, e, t0, p.tpi_dn, wi);
  wi.nt = nt;
  const int q = wi.q;
  const uint32_t lut_bytes = 256u << P.qmax;
  switch (q < 3 || q > P.qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3:  // pair tables (the launch holds their LDS, fused_lds_bytes)
      if (nt <= kDbTok) down_body<3, 1, true, true, true, true>(p, wi, it, lds, kPairTableBytes, tid, ksi);
      else down_body<3, 1, true, true, false, true>(p, wi, it, lds, kPairTableBytes, tid, ksi);
      break;
    case 4:
      if (nt <= kDbTok) down_body<4, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      else down_body<4, 1, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      break;
    case 5:
      if (nt <= kDbTok) down_body<5, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      else down_body<5, 1, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      break;
    case 6:
      if (nt <= kDbTok) down_body<6, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      else down_body<6, 1, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      break;
    case 7:
      if (nt <= kDbTok) down_body<7, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      else down_body<7, 1, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      break;
    case 8:
      if (nt <= kDbTok) down_body<8, 1, true, true, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      else down_body<8, 1, true>(p, wi, it, lds, lut_bytes, tid, ksi);
      break;
    default: poison_y(p, ksi, wi.base, nt, it * 128);
  }
  mark_done(ctr(P, C_DOWN));
}

// bf16 -> fp16 conversion of token t: its scale shift (largest finite
// exponent, reduced through LDS bytes 64..95, clear of the unit slot), then
// the scaled conversion, as k_x_to_f16 does.
__device__ __forceinline__ void conv_unit(const FusedParams& P, int t, uint16_t* lds, int tid) {
  const FfnParams& p = P.f;
  int* red = (int*)((char*)lds + 64);
  const int n8 = p.H / 8;
  const uint16_t* xr = P.x + (size_t)t * p.H;
  int m = 0;
  for (int i = tid; i < n8; i += kThreads) m = max(m, max_exp8_bf16(xr + 8 * i));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  int mx = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mx = max(mx, red[w]);
  const int shift = x_scale_shift(mx);
  if (tid == 0) st_co<true>(const_cast<int32_t*>(p.xsc) + t, shift);
  for (int i = tid; i < n8; i += kThreads)
    st_co16<true>((uint16_t*)p.xh + (size_t)t * p.H + 8 * i, __builtin_bit_cast(uint4, load_x8_bf16(xr + 8 * i, shift)));
  mark_done(ctr(P, C_CONV));
}

template <int XDT>
__device__ __forceinline__ void logit_unit(const FusedParams& P, int u, uint16_t* lds, int tid) {
  const FfnParams& p = P.f;
  const int lane = tid & 63, w = tid >> 6;
  const long long wu = (long long)u * 8 + w;
  if (P.logit_mfma) {
    logits_tile_mfma<XDT, true>(P.x, P.W, p.T, p.H, p.E, wu, lane, P.logits, route_ws_l1(P.logits, 1, p.T, p.E));
  } else {
    double* part = (double*)lds + w * (kTT * 65);
    logits_partials<XDT, 1, 2, true>(P.x, P.W, p.T, p.H, p.E, P.ks, wu, lane, part,
                                     route_ws_l1(P.logits, P.ks, p.T, p.E));
    __syncthreads();
    logits_sum<1, true>(p.T, p.E, P.ks, wu, lane, part, P.logits);
  }
  mark_done(ctr(P, C_LOGIT));
}

template <int XDT>
__device__ __forceinline__ void topk_unit(const FusedParams& P, int u, uint16_t* lds, uint32_t* flag, int tid) {
  const FfnParams& p = P.f;
  const int lane = tid & 63, w = tid >> 6;
  if (wait_count(P, C_LOGIT, P.n_logit, flag)) {
    // LDS: lg [8][512] fp64, sel_v [8][17] fp64, sel_i [8][17], the norm maximum, exact scratch [8]
    double* lg = (double*)lds + w * 512;
    double* sel_v = (double*)lds + 8 * 512 + w * 17;
    int* sel_i = (int*)((double*)lds + 8 * 512 + 8 * 17) + w * 17;
    unsigned* nmax = (unsigned*)((int*)((double*)lds + 8 * 512 + 8 * 17) + 8 * 17);
    ExactScratch* sc = (ExactScratch*)((char*)nmax + 16) + w;
    const int t = u * 8 + w;
    if (tid == 0) *nmax = 0u;
    __syncthreads();
    const float xi = topk_gather<XDT, true>(P.logits, P.x, P.bias, P.ks, t, p.T, p.H, p.E, lane, tid, kThreads, lg,
                                            nmax);
    topk_load<true>(P.logits, P.bias, P.ks, t, p.T, p.E, lane, lg);
    __syncthreads();
    topk_rank(t, p.T, p.E, p.K, lane, lg, sel_v, sel_i);
    __syncthreads();
    topk_certify<XDT>(P.x, P.W, P.bias, t, p.T, p.H, p.E, p.K, lane, lg,
                      logit_bound(p.H, xi, __uint_as_float(*nmax)), sel_v, sel_i, *sc);
    topk_finish<true>(t, p.T, p.K, lane, sel_v, sel_i, P.idx_out, P.w_out);
  }
  mark_done(ctr(P, C_TOPK));
}

__device__ __forceinline__ void comb_unit(const FusedParams& P, int u, uint32_t* flag, int tid) {
  const FfnParams& p = P.f;
  bool ok = wait_count(P, C_GROUP, P.n_group, flag);
  if (ok) ok = wait_count(P, C_DOWN, (uint32_t)p.n_items[1] * P.ntile_dn * p.dn_split, flag);
  const size_t H4 = p.H >> 2, gid = (size_t)u * 512 + tid;
  if (gid < (size_t)p.T * H4) {
    const int t = (int)(gid / H4), n = (int)(gid - (size_t)t * H4) * 4;
    if (ok) combine4<true>(p, t, n);
    else *(f32x4*)(p.out + (size_t)t * p.H + n) = (f32x4){__builtin_nanf(""), __builtin_nanf(""),
                                                          __builtin_nanf(""), __builtin_nanf("")};
  }
}

// Takes the next unit (whole workgroup) and returns it.
__device__ __forceinline__ uint32_t next_unit(const FusedParams& P, uint32_t* slot) {
  __syncthreads();  // the previous unit is finished with LDS and the slot
  if (threadIdx.x == 0)
    slot[0] = __hip_atomic_fetch_add(ctr(P, C_HEAD), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t u = __builtin_amdgcn_readfirstlane(slot[0]);
  __syncthreads();  // read by every wave before a unit may write LDS byte 0
  return u;
}

// An opaque copy of the thread index: nothing derived from it is hoisted out
// of a unit loop, so a unit's registers are live during that unit only.
__device__ __forceinline__ int opaque_tid() {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  return tid & (kThreads - 1);  // keeps the known range for address arithmetic
}

// The parameters, read again from the kernel argument segment for each unit:
// nothing loaded from them is kept across units, which keeps the scalar
// registers of one unit free for that unit.
__device__ __forceinline__ FusedParams unit_params() {
#if __HIP_DEVICE_COMPILE__
  typedef const __attribute__((address_space(4))) FusedParams* kparams_t;
  kparams_t k = (kparams_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(k));
  return *k;
#else
  return FusedParams{};  // device-only function; the host pass only parses it
#endif
}

template <int XDT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_fused(FusedParams P) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  uint32_t* slot = (uint32_t*)((char*)lds + P.slot_off);  // [0] unit, [1] error flag
  uint32_t* flag = slot + 1;
  // units are taken in increasing order, so each phase is one loop and a
  // workgroup never returns to an earlier phase
  const uint32_t b_logit = P.n_conv, b_topk = b_logit + P.n_logit, b_group = b_topk + P.n_topk,
                 b_gu = b_group + P.n_group, b_dn = b_gu + P.n_gu, b_comb = b_dn + P.n_dn, b_end = b_comb + P.n_comb;
  uint32_t u = next_unit(P, slot);
  for (; u < b_logit; u = next_unit(P, slot)) conv_unit(unit_params(), (int)u, lds, opaque_tid());
  for (; u < b_topk; u = next_unit(P, slot)) logit_unit<XDT>(unit_params(), (int)(u - b_logit), lds, opaque_tid());
  for (; u < b_group; u = next_unit(P, slot)) topk_unit<XDT>(unit_params(), (int)(u - b_topk), lds, flag, opaque_tid());
  for (; u < b_gu; u = next_unit(P, slot)) {
    const FusedParams Q = unit_params();
    const int tid = opaque_tid();
    if (wait_count(Q, C_TOPK, Q.n_topk, flag)) group_unit(Q.f, (int)(u - b_group), (int*)lds, tid);
    mark_done(ctr(Q, C_GROUP));
  }
  for (; u < b_dn; u = next_unit(P, slot)) {
    const FusedParams Q = unit_params();
    const int tid = opaque_tid();
    if (wait_count(Q, C_GROUP, Q.n_group, flag) && wait_count(Q, C_CONV, Q.n_conv, flag))
      gate_up_unit(Q, (int)(u - b_gu), lds, slot, tid);
  }
  for (; u < b_comb; u = next_unit(P, slot)) {
    const FusedParams Q = unit_params();
    const int tid = opaque_tid();
    if (wait_count(Q, C_GROUP, Q.n_group, flag)) down_unit(Q, (int)(u - b_dn), lds, slot, tid);
  }
  for (; u < b_end; u = next_unit(P, slot)) comb_unit(unit_params(), (int)(u - b_comb), flag, opaque_tid());
  // the last workgroup out leaves the counters at zero for the next launch
  if (threadIdx.x == 0) {
    const uint32_t n = __hip_atomic_fetch_add(ctr(P, C_EXIT), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (n == gridDim.x - 1)
      for (int i = 0; i < C_GU + P.f.NB; ++i)
        __hip_atomic_store(ctr(P, i), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

size_t fused_lds_bytes(int qmax) {
  const size_t ffn = std::max<size_t>(std::max<size_t>((256u << qmax) + stage_bytes<1>(), kWaves * 16 * 64 * 4),
                                      kPairTableBytes + stage_bytes<1>());
  const size_t logit = 8 * kTT * 65 * 8;
  constexpr size_t topk = 8 * 512 * 8 + 8 * 17 * 8 + 8 * 17 * 4 + 16 + 8 * sizeof(ExactScratch);
  static_assert(topk <= kPairTableBytes + stage_bytes<1>(), "the router units fit the smallest FFN LDS");
  const size_t grp = (kMaxGroupsF + 48) * 4;
  return (std::max(std::max(ffn, logit), std::max(topk, grp)) + 255) / 256 * 256;
}

}  // namespace

size_t fused_counter_bytes() { return (size_t)(C_GU + kMaxGroupsF) * kCtrStride * 4; }

hipError_t launch_fused(const FusedLaunch& L, hipStream_t s) {
  FusedParams P{};
  P.f = L.f;
  P.x = L.x;
  P.W = L.W;
  P.bias = L.bias;
  P.logits = L.logits;
  P.idx_out = L.idx_out;
  P.w_out = L.w_out;
  P.ctr = L.ctr;
  P.qmax = L.qmax;
  const FfnParams& f = L.f;
  const long long ntt = (f.T + kTT - 1) / kTT;
  P.n_conv = L.xdt == 1 ? f.T : 0;  // one unit per token
  P.logit_mfma = logits_use_mfma(f.T, f.E) ? 1 : 0;
  P.ks = route_ksplit(f.T, f.H, f.E);
  P.n_logit = P.logit_mfma ? (int)(((long long)((f.T + 15) / 16) * ((f.E + 15) / 16) + 7) / 8)
                           : (int)((ntt * f.E * P.ks + 7) / 8);
  P.n_topk = (f.T + 7) / 8;
  P.n_group = f.NB;
  P.ntile_gu = f.I >> 6;
  P.ntile_dn = (f.H + 127) >> 7;
  P.n_gu = f.max_items * P.ntile_gu;
  P.n_dn = f.max_items * P.ntile_dn * f.dn_split;
  P.n_comb = (int)(((long long)f.T * (f.H >> 2) + 511) / 512);
  // the unit slot and the wait flag sit at LDS byte 0: they are read before a
  // unit writes any LDS and rewritten only after the unit's last LDS access
  P.slot_off = 0;
  const size_t shmem = fused_lds_bytes(L.qmax);
  const void* fn = L.xdt == 1 ? (const void*)k_fused<1> : (const void*)k_fused<0>;
  static unsigned long long lds_raised[2] = {0, 0};  // per activation dtype: devices done
  hipError_t e = raise_lds_limit(fn, (int)fused_lds_bytes(8), lds_raised[L.xdt]);
  if (e != hipSuccess) return e;
  int per_cu = 0, dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, shmem);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const long long total = (long long)P.n_conv + P.n_logit + P.n_topk + P.n_group + P.n_gu + P.n_dn + P.n_comb;
  const unsigned grid = (unsigned)std::min<long long>(total, (long long)per_cu * cus);
  if (L.xdt == 1) hipLaunchKernelGGL(k_fused<1>, dim3(grid), dim3(kThreads), shmem, s, P);
  else hipLaunchKernelGGL(k_fused<0>, dim3(grid), dim3(kThreads), shmem, s, P);
  return hipGetLastError();
}

}  // namespace mpb
