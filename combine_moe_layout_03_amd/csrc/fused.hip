// Layout + notify + dispatch in one launch: the single-kernel, low-latency
// form of the EP pipeline ("UMDK/CAM communication acceleration library deep
// analysis v2", section 3.2, moe_dispatch_lowlatency_zb: local expert counts,
// count exchange, global count matrix and prefix sum, then the token writes,
// all inside one kernel), with the stage definitions of sections 2.3-2.5.
// Results are identical to moe_layout, moe_notify and moe_dispatch called in
// turn.
//
// The pages' kernel synchronises its cores between the phases.  On one
// MI355X a grid-wide barrier costs more than the work it would save: every
// workgroup's arrival is a device-scope atomic on one address, and 256-512 of
// them serialise at the memory side, tens of microseconds.  Counting the ids
// is cheap next to the rows, so here every workgroup counts all of them
// itself and no workgroup waits on another.  A workgroup's 16 waves split
// into 8 counting waves and 8 row waves:
//   1. The counting waves issue the loads of all their ids; after a
//      workgroup barrier, each row wave issues the loads of its first
//      token's row (up to 14 chunks per lane, h <= 7168; a longer row
//      follows step 4), which arrive while steps 2-4 run.  Tokens go to the
//      row waves first, so a group of up to 8 tokens has all its rows
//      early.  Issuing a row's 14 loads stalls a wave for as long as the
//      memory system takes to accept them (up to about 10 us at bs 4096,
//      h 7168), so the row waves do nothing else until step 5.
//   2. The counting waves count all bs*k ids into two LDS histograms: the
//      entries before this workgroup's first entry, and the rest.  Their sum
//      is the layout stage's per-expert totals (with invalid ids in the last
//      bin).  Each histogram has C copies (lane l adds to copy l % C): lanes
//      of one atomic that hit the same expert hit at most 64 / C to one
//      word: with one copy, a batch that sends every entry to one expert
//      makes each atomic 64-way serial (about 18 us more at bs 4096); with
//      8 copies it costs what a uniform batch does.  The copies are summed
//      afterwards.
//   3. An exclusive scan of the totals in LDS is the notify stage: the
//      receive row of (expert e, slot s) is scan[e] + s.  The first
//      ceil(E / 64) counting waves (one expert per lane; up to 4 when
//      E > 512) scan; the other counting waves load their rows instead, as
//      the row waves did.  Workgroup 0 writes the layout and notify outputs.
//   4. The scanning waves rank the workgroup's own entries, rounds of 64
//      entries in turn: an entry's slot is its expert's count before the
//      workgroup plus the same-expert entries before it in the workgroup,
//      counted with match-any ballots over its own round and each earlier
//      one, so the rounds are independent (its stable rank within its
//      expert).  The slots go to LDS and to sendTokenIdx.
//   The counting waves synchronise steps 2-3 among themselves through LDS
//   counters; a workgroup barrier after step 4 lets every wave on.
//   5. Each wave quantises (or passes through) its tokens and writes every
//      copy, as the dispatch kernel does; the scanning waves load their rows
//      here.
// The ids are read once per workgroup from L2 (bs*k*4 bytes each); with one
// workgroup per CU that is the only redundant work.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "launch.h"
#include "quant.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kFusedWaves;
constexpr int kThreads = kWaves * kWave;
constexpr int kCountWaves = kWaves / 2;  // waves that count the ids
constexpr int kCountThreads = kCountWaves * kWave;
constexpr int kQuads = 16;  // groups of four ids per counting thread and round
constexpr int kSyncs = 2;   // sync points of the counting waves: ids counted, scan sums
constexpr int kMaxCopies = 1 << kFusedMaxCopiesLog2;
constexpr int kMaxIdBits = 11;  // bits of an expert id (E <= 2048)
static_assert(MOE_MAX_EXPERTS <= (1 << kMaxIdBits), "expert ids fit in kMaxIdBits bits");
constexpr int kMaxPer = 4;  // experts per scanning lane (at E = 2048)
constexpr int kScanExpertsPerWave = kMaxPer * kWave;
static_assert(MOE_MAX_EXPERTS <= kScanExpertsPerWave * kCountWaves, "the counting waves can scan every expert");
// s_waitcnt vmcnt(0) with expcnt and lgkmcnt at their maxima.  The compiler
// places its waits for loads per register, merging the two paths below as
// if either could have run: the ids' registers look in flight on the row
// path, and the row's on the id path, so code after the paths join would
// wait there for part of the row.  An explicit wait on each path, where
// nothing is in flight in fact, clears that state.
constexpr int kWaitVm0 = 0x0f70;

// Row t into registers, 16 bytes (8 elements) per chunk, chunk lane + 64 i
// in v[i].  Chunks past the row's end load its last chunk again (a duplicate
// changes no maximum and is never stored), so every load is unconditional.
// The loads are non-temporal (a row is read once): about 0.5-1 us faster at
// bs 4096, h 7168 than ordinary loads.  (Non-temporal stores of the receive
// rows were 27 us slower: the rows are scattered, and ordinary stores let
// the Infinity Cache gather them.)
template <int kVpl>
__device__ __forceinline__ void load_row(uint4 (&v)[kVpl], const uint16_t* x, int t, int hidden, int lane) {
  const uint32_t last = static_cast<uint32_t>(hidden >> 3) - 1u;
  const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * hidden);
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const uint32_t c = static_cast<uint32_t>(lane + i * kWave);
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (c < last ? c : last)));
    v[i] = make_uint4(w.x, w.y, w.z, w.w);
  }
}

template <bool kFp16, bool kQuant, int kVpl>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedArgs a) {
  extern __shared__ int32_t lds[];
  const int E = a.num_experts;
  const int C = 1 << a.copies_log2;       // histogram copies: lane l counts into copy l % C
  // Copy c of bin e at [c * (E + 1) + e]: summing the copies of a bin, the
  // lanes of a wave read consecutive words (a bin-major layout made that
  // read 8-way bank-conflicted, 1.2 us at 8 copies).
  int32_t* hpre = lds;                    // [C][E + 1] copies of the counts before this group
  int32_t* htot = hpre + (E + 1) * C;     // [C][E + 1] copies of the counts from this group on
  int32_t* pre = htot + (E + 1) * C;      // [E + 1] counts before this group
  int32_t* tot = pre + (E + 1);           // [E + 1] totals (tot[E]: invalid ids)
  int32_t* gsc = tot + (E + 1);           // [E + 1] exclusive scan of the totals (gsc[E]: all valid)
  int32_t* ids_l = gsc + (E + 1);         // [T * k] own entries' ids
  int32_t* slot_l = ids_l + a.tokens_per_group * a.k;  // [T * k] own entries' slots (-1: dropped)
  __shared__ int32_t wave_sum[kCountWaves];
  __shared__ int32_t sync_ctr[kSyncs];  // counting-wave arrivals per sync point

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid / kWave);
  const int group = blockIdx.x;
  const int n = a.bs * a.k;  // at most kFusedMaxEntries
  const int t_begin = min(group * a.tokens_per_group, a.bs);
  const int t_end = min(t_begin + a.tokens_per_group, a.bs);
  const int e_begin = t_begin * a.k;
  const int own = (t_end - t_begin) * a.k;

  // 1-2. Histograms of all ids, by the counting waves 0 .. kCountWaves - 1:
  //      before this group's first entry, and the rest; the group's own ids
  //      are also kept in LDS.  A counting thread reads kQuads groups of four
  //      ids per round (16-byte loads when the ids are 16-byte aligned),
  //      indices clamped to the last whole group and the loads issued back to
  //      back; the last n % 4 ids are counted one by one.
  //      The other waves (the row waves) load their first tokens' rows
  //      meanwhile, asked for after the counting waves' ids, which then
  //      arrive first.  A wave stalls while its row's loads wait to issue,
  //      which lasts until most rows are in (about 10 us at bs 4096,
  //      h 7168); so the row waves take no part in the count, the scan or
  //      the ranking, and those phases synchronise only the counting waves,
  //      through LDS counters.  The row waves go on at the workgroup barrier
  //      after the ranking.
  const int copy = lane & (C - 1);
  const bool counter = wave < kCountWaves;
  const int nq = n >> 2;  // whole groups of four ids
  const int hist_pre = copy * (E + 1);          // this lane's copy in hpre
  const int hist_tot = hist_pre + (E + 1) * C;  // and in htot, which follows hpre
  auto count_one = [&](int i, int e) {
    const int bin = static_cast<int>(min(static_cast<unsigned>(e), static_cast<unsigned>(E)));  // invalid: E
    atomicAdd(hpre + (i < e_begin ? hist_pre : hist_tot) + bin, 1);
  };
  int4 quads[kQuads];
  // A wave whose first group of the round is past the last loads nothing
  // (its later groups are further on).
  auto load_round = [&](int q0) {
    if (q0 + wave * kWave >= nq) return;
    if (a.ids_aligned16) {
      const int4* src = reinterpret_cast<const int4*>(a.topk_idx);
#pragma unroll
      for (int u = 0; u < kQuads; ++u) quads[u] = src[min(q0 + u * kCountThreads + tid, nq - 1)];
    } else {
#pragma unroll
      for (int u = 0; u < kQuads; ++u) {
        const int32_t* src = a.topk_idx + 4 * min(q0 + u * kCountThreads + tid, nq - 1);
        quads[u] = make_int4(src[0], src[1], src[2], src[3]);
      }
    }
  };
  auto count_round = [&](int q0) {
    if (q0 + wave * kWave >= nq) return;
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int q = q0 + u * kCountThreads + tid;
      if (q < nq) {
        count_one(4 * q, quads[u].x);
        count_one(4 * q + 1, quads[u].y);
        count_one(4 * q + 2, quads[u].z);
        count_one(4 * q + 3, quads[u].w);
      }
    }
  };
  // Sync point p among some of the counting waves: each arrives once (its
  // LDS writes before the arrival are seen after the wait), and a waiting
  // wave goes on once `count` waves have arrived.  Every wave a wait counts
  // on arrives unconditionally (the kernel has no early exit, and a
  // workgroup's waves are resident together), so each wait ends.
  auto counters_arrive = [&](int p) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(&sync_ctr[p], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto counters_wait = [&](int p, int count) {
    while (__hip_atomic_load(&sync_ctr[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < count) {
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  constexpr int kRound = kCountThreads * kQuads;  // groups of four per round
  // The group's own ids (for the ranking) are read beside the first round.
  const bool own_first = counter && tid < own;
  const int own_id = own_first ? a.topk_idx[e_begin + tid] : 0;
  if (counter && nq > 0) load_round(0);
  for (int e = tid; e < 2 * (E + 1) * C; e += kThreads) hpre[e] = 0;  // hpre and htot
  if (tid < kSyncs) sync_ctr[tid] = 0;
  __syncthreads();
  // The first token of this wave.
  uint4 v[kVpl];
  // Tokens go to the row waves first: wave w takes the group's tokens
  // (w - kCountWaves) mod kWaves, then every kWaves-th after it, so a group
  // of at most kWaves - kCountWaves tokens has all its rows loaded early.
  const int t_first = t_begin + (wave + kWaves - kCountWaves) % kWaves;
  // A row of up to 14 chunks per lane (h <= 7168) is loaded early; a
  // longer one would not fit in registers beside a counting wave's ids (the
  // kernel's register budget covers both kinds of wave) and is loaded after
  // the barrier.
  constexpr bool kRowDuringCount = kVpl <= 14;
  // Waves 0 .. scan_waves - 1 scan (one expert per lane, at most 4 when
  // E > 512) and rank; every other wave loads its row early.
  const int scan_waves = min(kCountWaves, (E + kWave - 1) / kWave);
  const bool scanner = wave < scan_waves;
  const bool have_row = kRowDuringCount && !scanner;
  if (counter) {
    if (nq > 0) count_round(0);
    for (int q0 = kRound; q0 < nq; q0 += kRound) {
      load_round(q0);
      count_round(q0);
    }
    const int i = 4 * nq + tid;
    if (i < n) count_one(i, a.topk_idx[i]);
    if (own_first) ids_l[tid] = own_id;
    for (int li = tid + kCountThreads; li < own; li += kCountThreads) ids_l[li] = a.topk_idx[e_begin + li];
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // ids that no lane used
    counters_arrive(0);
  }
  if (scanner) {
    counters_wait(0, kCountWaves);

    // 3. Totals and their exclusive scan (notify).  Scanning thread c owns
    //    the contiguous experts [c * per, (c + 1) * per), per <= kMaxPer,
    //    sums their histogram copies and scans; the last scanning thread
    //    also sums the invalid-id bin E.
    // The C copies of bin e summed: all kMaxCopies reads are issued at once
    // (copy indices clamped to C - 1, the extra reads not added); reads
    // guarded one by one waited for each other, about 1 us per scan.
    auto sum_copies = [&](int e, int& sp, int& st) {
      int vp[kMaxCopies], vt[kMaxCopies];
#pragma unroll
      for (int c = 0; c < kMaxCopies; ++c) {
        const int cc = min(c, C - 1);
        vp[c] = hpre[cc * (E + 1) + e];
        vt[c] = htot[cc * (E + 1) + e];
      }
#pragma unroll
      for (int c = 0; c < kMaxCopies; ++c) {
        sp += c < C ? vp[c] : 0;
        st += c < C ? vt[c] : 0;
      }
    };
    const int scan_threads = scan_waves * kWave;
    const int per = (E + scan_threads - 1) / scan_threads;  // <= kMaxPer
    const int e0 = tid * per;
    int cnt[kMaxPer];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      cnt[q] = 0;
      const int e = e0 + q;
      if (q < per && e < E) {
        int sp = 0, st = 0;
        sum_copies(e, sp, st);
        pre[e] = sp;
        cnt[q] = sp + st;
        sum += cnt[q];
      }
    }
    if (tid == scan_threads - 1) {
      int sp = 0, st = 0;
      sum_copies(E, sp, st);
      tot[E] = sp + st;
    }
    const int incl = wave_inclusive_scan(sum);
    int off = 0;
    int total = incl;  // one scanning wave: its last lane's sum
    if (scan_waves > 1) {
      if (lane == kWave - 1) wave_sum[wave] = incl;
      counters_arrive(1);
      counters_wait(1, scan_waves);
      total = 0;
      int ws[kCountWaves];  // all reads at once, as in sum_copies
#pragma unroll
      for (int w = 0; w < kCountWaves; ++w) ws[w] = wave_sum[min(w, scan_waves - 1)];
#pragma unroll
      for (int w = 0; w < kCountWaves; ++w) {
        off += w < wave ? ws[w] : 0;
        total += w < scan_waves ? ws[w] : 0;
      }
    } else {
      total = __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    int excl = off + incl - sum;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      const int e = e0 + q;
      if (q < per && e < E) {
        tot[e] = cnt[q];
        gsc[e] = excl;
        excl += cnt[q];
      }
    }
    if (tid == scan_threads - 1) gsc[E] = total;

    // 4. Slots of this group's own entries: entry li's slot is its expert's
    //    count before the group (pre) plus the entries of the same expert
    //    before it in the group.  Rounds of 64 entries go to the scanning
    //    waves in turn (wave w: rounds w, w + scan_waves, ...), each round
    //    on its own: match-any ballots over the round give the same-expert
    //    lanes below, and over each earlier round the same-expert entries
    //    there, so no round waits for another.
    for (int r = wave; r * kWave < own; r += scan_waves) {
      const int li = r * kWave + lane;
      const bool in_range = li < own;
      const int e = in_range ? ids_l[li] : -1;
      const bool valid = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(E);
      // lanes whose entry (of round r2's ids `e2`) has this lane's expert
      auto same_expert = [&](int e2, bool valid2) {
        uint64_t m = __ballot(valid2);
#pragma unroll
        for (int bit = 0; bit < kMaxIdBits; ++bit) {
          if (bit < a.id_bits) {
            const uint64_t set = __ballot((e2 >> bit) & 1);
            m &= ((e >> bit) & 1) ? set : ~set;
          }
        }
        return m;
      };
      int before = valid ? lanes_below(same_expert(e, valid)) : 0;
      for (int r2 = 0; r2 < r; ++r2) {
        const int e2 = ids_l[r2 * kWave + lane];  // an earlier round is whole
        const uint64_t m = same_expert(e2, static_cast<unsigned>(e2) < static_cast<unsigned>(E));
        before += valid ? __popcll(m) : 0;
      }
      if (in_range) {
        const int slot = valid ? pre[e] + before : -1;
        slot_l[li] = slot;
        a.send_token_idx[e_begin + li] = slot;
      }
    }
  } else if (kRowDuringCount && t_first < t_end) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // nothing in flight here: free
    load_row<kVpl>(v, a.x, t_first, a.hidden, lane);
  }
  // The waves that load their rows early are here at the latest when those
  // loads have issued; the scanning waves once the slots are ranked.  (Held
  // at this barrier, no wave starts its stores before every early row's
  // loads have issued: with an LDS flag instead, stores that began once the
  // slots were ready kept some rows' loads from issuing for up to 20 us.)
  __syncthreads();
  if (group == 0 && counter) {
    for (int e = tid; e < E; e += kCountThreads) {
      const int first = (e / a.epr) * a.epr;
      a.token_per_expert[e] = tot[e];
      a.recv_token_per_expert[e] = tot[e];
      a.put_offset[e] = gsc[e] - gsc[first];
    }
    for (int r = tid; r < a.ranks; r += kCountThreads) {
      const int c = gsc[(r + 1) * a.epr] - gsc[r * a.epr];
      a.recv_base[r] = gsc[r * a.epr];
      a.recv_count[r] = c;
      a.token_per_rank[r] = c;
    }
    if (tid == 0 && a.bad_count != nullptr) *a.bad_count = tot[E];
  }

  // 5. Dispatch of this group's tokens: wave w takes tokens w, w + 16, ...
  const int chunks = a.hidden >> 3;
  for (int t = t_first; t < t_end; t += kWaves) {
    if (t != t_first || !have_row) load_row<kVpl>(v, a.x, t, a.hidden, lane);
    const int li0 = (t - t_begin) * a.k;
    if constexpr (!kQuant) {
      for (int j = 0; j < a.k; ++j) {
        const int slot = slot_l[li0 + j];
        if (slot < 0) continue;
        const int64_t row = static_cast<int64_t>(gsc[ids_l[li0 + j]]) + slot;  // recvBase[rank] + putOffset[e]
        if (row >= a.cap_rows) continue;
        u32x4* dst = reinterpret_cast<u32x4*>(a.recv + row * a.row_bytes);
        // Element-wise vector stores: a whole-struct uint4 copy here is a
        // 16-byte memcpy out of v, which kept v in scratch memory (240 bytes
        // per lane at h = 7168) and doubled the passthrough time.
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
          const int c = lane + i * kWave;
          if (c < chunks) dst[c] = u32x4{v[i].x, v[i].y, v[i].z, v[i].w};
        }
      }
    } else {
      u16x2 m2 = {0, 0};
#pragma unroll
      for (int i = 0; i < kVpl; ++i) m2 = max_magnitude(m2, v[i]);
      const uint32_t m = wave_max_u32(m2.x > m2.y ? m2.x : m2.y);
      float s, inv;
      row_scale<kFp16>(m, s, inv);
      uint2 q[kVpl];
#pragma unroll
      for (int i = 0; i < kVpl; ++i) q[i] = quantise_chunk<kFp16>(v[i], s);
      for (int j = 0; j < a.k; ++j) {
        const int slot = slot_l[li0 + j];
        if (slot < 0) continue;
        const int64_t row = static_cast<int64_t>(gsc[ids_l[li0 + j]]) + slot;
        if (row >= a.cap_rows) continue;
        uint8_t* base = a.recv + row * a.row_bytes;
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
          const int c = lane + i * kWave;
          if (c < chunks) reinterpret_cast<uint2*>(base)[c] = q[i];
        }
        if (lane == 0) *reinterpret_cast<float*>(base + a.scale_off) = inv;
      }
    }
  }
}

// One case per entry of select::kFusedVpl.
template <bool kFp16, bool kQuant>
const void* pick_kernel(int hidden) {
#define MOE_FUSED_CASE(V) \
  case V: return reinterpret_cast<const void*>(&fused_kernel<kFp16, kQuant, V>);
  switch (select::fused_vpl(hidden)) {
    MOE_FUSED_CASE(1)
    MOE_FUSED_CASE(2)
    MOE_FUSED_CASE(4)
    MOE_FUSED_CASE(8)
    MOE_FUSED_CASE(12)
    MOE_FUSED_CASE(14)
    MOE_FUSED_CASE(16)
  }
#undef MOE_FUSED_CASE
  return nullptr;
}

}  // namespace

size_t fused_lds_bytes(int32_t num_experts, int32_t tokens_per_group, int32_t topk, int32_t copies) {
  const size_t bins = static_cast<size_t>(num_experts) + 1;
  return ((2u * static_cast<size_t>(copies) + 3u) * bins + 2u * static_cast<size_t>(tokens_per_group) * topk) *
         sizeof(int32_t);
}

hipError_t launch_fused(const FusedArgs& a, Half x_type, bool quant, int groups, hipStream_t stream) {
  const void* f = nullptr;
  if (x_type == Half::kFp16) {
    f = quant ? pick_kernel<true, true>(a.hidden) : pick_kernel<true, false>(a.hidden);
  } else {
    f = quant ? pick_kernel<false, true>(a.hidden) : pick_kernel<false, false>(a.hidden);
  }
  if (f == nullptr || groups < 1) return hipErrorInvalidValue;
  const size_t lds = fused_lds_bytes(a.num_experts, a.tokens_per_group, a.k, 1 << a.copies_log2);
  FusedArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(f, dim3(groups), dim3(kThreads), args, lds, stream);
}

}  // namespace moe
