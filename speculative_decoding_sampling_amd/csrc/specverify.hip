// C ABI of libspecverify: argument checks, workspace layout and the launch
// sequence on the caller's stream.  The declarations and their contract live
// in include/specverify.h.
#include "specverify.h"
#include "specverify_selftest.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "accept_core.h"
#include "common.h"
#include "sample_core.h"

namespace specv {
int row_stats_chunk(bool bf16);
hipError_t launch_row_stats(bool bf16, const void* tgt, const void* dft, const int* draft_len,
                            const int* tokens, int B, int K, int V, int nchunk, float c,
                            float2* part, float* zx, hipStream_t stream, int row_lo = 0,
                            bool cached = false, bool pairs_only = false);
int lm_head_tiles(int V);
size_t lm_head_packed_elems(int V, int D);
hipError_t launch_lm_head_pack(const void* weight, void* packed, int V, int D,
                               hipStream_t stream);
int lm_head_rows_per_block();
int lm_head_kblock();
hipError_t launch_lm_head(const void* hidden, const void* weight, int M, int D, int V, float c,
                          void* logits, float2* tpart, hipStream_t stream);
hipError_t launch_fold_tile_stats(const float2* tpart, const void* logits, const int* tokens,
                                  int B, int K, int V, int nch, float c, float2* part, float* zx,
                                  hipStream_t stream);
hipError_t launch_accept(bool bf16, bool filt, const void* tgt, const void* dft, const int* tokens,
                         const int* draft_len, const float* u, const float* u_final, int B,
                         int K, int V, int nch_row, float c, double invT, int eos_id,
                         const float2* part, const float* zx, const FiltRow* frows,
                         const AcceptOut& out, hipStream_t stream);
int filter_cap(int top_k);
int filter_row_stride(int nch, int top_k);
hipError_t launch_filter(bool bf16, const void* tgt, const void* dft, const int* draft_len, int B,
                         int K, int V, int nch, int top_k, float top_p, double invT,
                         uint64_t* cand, int* counts, FiltRow* rows, Kept* kept, int* redo,
                         hipStream_t stream, hipEvent_t mid);
hipError_t launch_filter_rows(bool bf16, const void* tgt, const void* dft, const int* draft_len,
                              int B, int K, int V, int top_k, float top_p, double invT,
                              FiltRow* rows, Kept* kept, hipStream_t stream);
int stream_chunks(int V);
hipError_t launch_sample_list(bool bf16, const void* tgt, const void* dft, const float* u_final,
                              int B, int K, int V, double invT, const Plan* plan,
                              const FiltRow* rows, const Kept* kept, double2* cmass,
                              int* out_tokens, double* rmass_out, hipStream_t stream);
hipError_t launch_sample_pass(bool bf16, const void* tgt, const void* dft, int B, int K, int V,
                              int nch, double invT, const Plan* plan, ChunkRec* recs, Tie* ties,
                              hipStream_t stream);
hipError_t launch_sample_finish(bool bf16, const void* tgt, const void* dft, const float* u_final,
                                int B, int K, int V, int nch, double invT, const Plan* plan,
                                const ChunkRec* recs, const Tie* ties, int* out_tokens,
                                double* rmass_out, hipStream_t stream);
size_t small_blocks(int B, int K, int V);
int set_small_poll_limit(int limit);
bool small_fits(int K, int V, int nch_row);
hipError_t launch_verify_small(bool bf16, const void* tgt, const void* dft, const int* tokens,
                               const int* draft_len, const float* u, const float* u_final, int B,
                               int K, int V, int nch_row, float c, double invT, int eos_id,
                               uint64_t* part, uint64_t* zxw, ChunkRec* recs, Tie* ties,
                               PairStat* pstat, uint32_t* flags, uint32_t* calls,
                               const AcceptOut& out, hipStream_t stream);
hipError_t launch_exp64_selftest(const double* x, double* y, int n, hipStream_t stream);
hipError_t launch_beta(bool bf16, bool filt, const void* tgt, const void* dft,
                       const int* draft_len, int B, int K, int V, int nch_row, float c,
                       double invT, const float2* part, const FiltRow* frows, const Kept* kept,
                       float* beta_part, float* beta, hipStream_t stream);
hipError_t launch_round_stats(const int32_t* draft_tokens, const int32_t* draft_len,
                              const int32_t* out_tokens, const int32_t* n_emitted,
                              const float* beta, int B, int K, int32_t* accepted, float* expected,
                              long long* totals, hipStream_t stream);
size_t monitor_state_bytes(int B, int window);
hipError_t launch_monitor_reset(void* state, int B, int window, hipStream_t stream);
hipError_t launch_monitor_update(const int32_t* draft_tokens, const int32_t* draft_len,
                                 const int32_t* out_tokens, const int32_t* n_emitted, int B,
                                 int K, int max_k, int window, void* state,
                                 int32_t* next_draft_len, double* rate, hipStream_t stream);

// Kernel stages of one call, in launch order (specv_verify_timed records an
// event after each), by path: without filters; top-k / top-p through the
// candidate select (0 < top_k <= kFiltMaxTopK, candidates fitting the merge);
// top-k / top-p through the general radix select (every other setting);
// without filters at small sizes, through the one-kernel tail.
constexpr int kNumPaths = 4;
const char* const kStageNames[kNumPaths][4] = {
    {"row_stats", "accept", "sample_pass", "sample_finish"},
    {"filter_cand", "filter_merge", "accept", "sample_list"},
    {"filter_rows", "accept", "sample_list", nullptr},
    {"verify_small", nullptr, nullptr, nullptr}};
constexpr int kNumStages[kNumPaths] = {4, 4, 3, 1};

// Unfiltered calls with at most this many (request, row pair, 2048-token
// chunk) triples, B (K+1) ceil(V/2048), take the small-batch path
// (specv_set_small_batch_limit changes it).  Measured on MI355X: the
// one-kernel tail is ~5 us faster up to ~320 triples, even at ~380, and
// slower from ~600 on, where its per-workgroup L2 writebacks (one per
// arriving workgroup, serialised within an XCD) outgrow the launches saved.
constexpr long long kSmallBatchLimitDefault = 384;
std::atomic<long long> g_small_limit{kSmallBatchLimitDefault};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace regions, each 256-byte aligned.
// Without filters:
//   row partials   float2   [B][2K+1][nch_row]        (max, partial normaliser)
//   drafted logits float    [B][2K]                   (target rows, then draft rows)
//   beta partials  float    [B][K][nch_row]           (acceptance-rate chunk sums)
//   plans          Plan     [B]
//   chunk records  ChunkRec [B][nch_samp]             (fp64 sums per sampler chunk)
//   near ties      Tie      [B][nch_samp][kTieCap]
// and on the small-batch path (one kernel), the row partials as tagged words
// uint64 [B][2K+1][nch_row][2] and the drafted logits as tagged words uint64
// [B][2K] in place of the first two, chunk records and near ties
// [B][K+1][nch_samp](...) (the chunk pass runs for every row pair), plus
//   pair statistics PairStat [B][K+1]
//   pass flags      uint32   [B][K+1][nch_samp]
//   call counters   uint32   [B]               (never cleared: see small.hip)
// With top-k / top-p:
//   plans          Plan     [B]
//   candidates     uint64   [B][2K+1][row_stride]     (key, id); cap per chunk, >= 256 last
//   counts         int      [B][2K+1][nch_filt]
//   block-merge list int    [1 + B (2K+1)]            (count, then the rows)
//   filtered rows  FiltRow  [B][2K+1]
//   kept lists     Kept     [B][2K+1][kKeptCap]
struct Layout {
  bool filt = false;
  bool cand = false;         // filtered through the candidate select
  bool small = false;        // unfiltered, through the one-kernel tail
  int nch_row = 0, nch_samp = 0, nch_filt = 0, cap = 0;
  size_t off_row = 0, off_zx = 0, off_beta = 0, off_plan = 0, off_recs = 0, off_ties = 0;
  size_t off_cand = 0, off_counts = 0, off_redo = 0, off_frows = 0, off_kept = 0, off_cmass = 0;
  size_t off_pstat = 0, off_flags = 0, off_calls = 0, total = 0;
};

bool filters_on(int V, int top_k, float top_p) { return (top_k > 0 && top_k < V) || top_p < 1.0f; }

// The candidate select serves a small active top-k whose per-chunk slots fit
// the merge's on-chip list; every other filtered call takes the radix select.
bool candidate_path(int V, int top_k) {
  if (!(top_k > 0 && top_k < V && top_k <= kFiltMaxTopK)) return false;
  const int nch = (V + kFiltChunk - 1) / kFiltChunk;
  return nch <= kFiltMaxChunks && filter_row_stride(nch, top_k) <= kFiltSortMax;
}

// An unfiltered call small enough for the one-kernel path (its row partials
// counted for float32 rows, the smaller chunks: the same answer for either
// dtype).
bool small_path(int B, int K, int V) {
  const int ch = row_stats_chunk(false);
  const long long triples = (long long)B * (K + 1) * ((V + kSampChunk - 1) / kSampChunk);
  return small_blocks(B, K, V) > 0 && small_fits(K, V, (V + ch - 1) / ch) &&
         triples <= g_small_limit.load(std::memory_order_relaxed);
}

// Stage-table index of a call: 0 unfiltered, 1 candidate select, 2 radix
// select, 3 unfiltered through the one-kernel small-batch path.
int path_kind(int B, int K, int V, int top_k, float top_p) {
  if (!filters_on(V, top_k, top_p)) return small_path(B, K, V) ? 3 : 0;
  return candidate_path(V, top_k) ? 1 : 2;
}

// allow_small = false keeps an unfiltered call on the four-kernel layout
// (the fused LM-head call, which runs those kernels whatever the size).
Layout make_layout(int B, int K, int V, bool bf16, int top_k, float top_p,
                   bool allow_small = true) {
  Layout L;
  const size_t R = (size_t)(2 * K + 1);
  size_t off = 0;
  L.filt = filters_on(V, top_k, top_p);
  if (!L.filt) {
    L.small = allow_small && small_path(B, K, V);
    const size_t pairs = L.small ? (size_t)(K + 1) : 1;   // chunk-pass row pairs per request
    const int ch = row_stats_chunk(bf16);
    L.nch_row = (V + ch - 1) / ch;
    L.nch_samp = L.small ? (V + kSmallChunk - 1) / kSmallChunk : (V + kSampChunk - 1) / kSampChunk;
    L.off_row = off;
    off = align_up(off + (size_t)B * R * L.nch_row * (L.small ? 2 * sizeof(uint64_t) : sizeof(float2)));
    L.off_zx = off;
    off = align_up(off + (size_t)B * 2 * K * (L.small ? sizeof(uint64_t) : sizeof(float)));
    L.off_beta = off;
    off = align_up(off + (size_t)B * K * L.nch_row * sizeof(float));
    L.off_plan = off;
    off = align_up(off + (size_t)B * sizeof(Plan));
    L.off_recs = off;
    off = align_up(off + (size_t)B * pairs * L.nch_samp * sizeof(ChunkRec));
    L.off_ties = off;
    off = align_up(off + (size_t)B * pairs * L.nch_samp * kTieCap * sizeof(Tie));
    if (L.small) {
      L.off_pstat = off;
      off = align_up(off + (size_t)B * pairs * sizeof(PairStat));
      L.off_flags = off;
      off = align_up(off + (size_t)B * pairs * L.nch_samp * sizeof(uint32_t));
      L.off_calls = off;
      off = align_up(off + (size_t)B * sizeof(uint32_t));
    }
  } else {
    L.cand = candidate_path(V, top_k);
    L.off_plan = off;
    off = align_up(off + (size_t)B * sizeof(Plan));
    if (L.cand) {
      L.nch_filt = (V + kFiltChunk - 1) / kFiltChunk;
      L.cap = filter_cap(top_k);
      L.off_cand = off;
      off = align_up(off + (size_t)B * R * filter_row_stride(L.nch_filt, top_k) * sizeof(uint64_t));
      L.off_counts = off;
      off = align_up(off + (size_t)B * R * L.nch_filt * sizeof(int));
      L.off_redo = off;
      off = align_up(off + (1 + (size_t)B * R) * sizeof(int));
    }
    L.off_frows = off;
    off = align_up(off + (size_t)B * R * sizeof(FiltRow));
    L.off_kept = off;
    off = align_up(off + (size_t)B * R * kKeptCap * sizeof(Kept));
    if (!L.cand) {
      L.off_cmass = off;
      off = align_up(off + (size_t)B * stream_chunks(V) * sizeof(double2));
    }
  }
  L.total = off;
  return L;
}

specv_status_t check_sizes(int B, int K, int V, specv_dtype_t dtype, int top_k, float top_p) {
  if (B < 1 || K < 0 || K > SPECV_MAX_K || V < 1) return SPECV_EINVAL;
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_EINVAL;
  if (top_k < 0) return SPECV_EINVAL;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return SPECV_EINVAL;
  // B * (K+1) * V elements must index without overflow.
  if ((double)B * (double)(K + 1) * (double)V > 4.0e18) return SPECV_EINVAL;
  if (V > SPECV_MAX_V) return SPECV_EUNSUPPORTED;
  if ((size_t)B * (2 * K + 1) * (size_t)((V + 1023) / 1024) > 0x7fffffffu) return SPECV_EUNSUPPORTED;
  return SPECV_OK;
}

bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

specv_status_t run(const void* target, const void* draft, specv_dtype_t dtype,
                   const int32_t* tokens, const int32_t* draft_len, const float* u,
                   const float* u_final, int B, int K, int V, float temperature, int top_k,
                   float top_p, int eos_id, int32_t* out_tokens, int32_t* n_emitted,
                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                   float* alpha_out, double* rmass_out, int32_t* stop_out, int32_t* path_out,
                   hipEvent_t* events, bool sampling = false) {
  specv_status_t st = check_sizes(B, K, V, dtype, top_k, top_p);
  if (st != SPECV_OK) return st;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SPECV_EINVAL;
  if (eos_id < -1 || eos_id >= V) return SPECV_EINVAL;
  const size_t esz = dtype == SPECV_BF16 ? 2 : 4;
  // A sampling call is a verification with no drafts: draft_len and
  // n_emitted may then be null (every request draws its bonus token).
  if (sampling && K != 0) return SPECV_EINVAL;
  if (!target || !u_final || !out_tokens) return SPECV_EINVAL;
  if (!sampling && (!draft_len || !n_emitted)) return SPECV_EINVAL;
  if (K > 0 && (!draft || !tokens || !u)) return SPECV_EINVAL;
  if (misaligned(target, esz) || (draft && misaligned(draft, esz))) return SPECV_EINVAL;
  if (misaligned(draft_len, 4) || misaligned(u_final, 4) || misaligned(out_tokens, 4) ||
      misaligned(n_emitted, 4) || (tokens && misaligned(tokens, 4)) || (u && misaligned(u, 4)))
    return SPECV_EINVAL;
  if ((alpha_out && misaligned(alpha_out, 4)) || (rmass_out && misaligned(rmass_out, 8)) ||
      (stop_out && misaligned(stop_out, 4)) || (path_out && misaligned(path_out, 4)))
    return SPECV_EINVAL;
  const bool bf16 = dtype == SPECV_BF16;
  const Layout L = make_layout(B, K, V, bf16, top_k, top_p);
  if (!workspace || misaligned(workspace, 16) || workspace_bytes < L.total) return SPECV_EWORKSPACE;

  char* ws = static_cast<char*>(workspace);
  Plan* plan = reinterpret_cast<Plan*>(ws + L.off_plan);

  // log2(e) / T rounded once to float32; every float32 exponent uses it.
  const float c = (float)(1.4426950408889634 / (double)temperature);
  const double invT = 1.0 / (double)temperature;

  // Events (timing variant only): events[0] before the first launch, events[i+1]
  // after stage i.
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord(events[i], stream) == hipSuccess;
  };
  if (!mark(0)) return SPECV_EHIP;
  hipError_t e;
  AcceptOut out;
  out.plan = plan;
  out.out_tokens = out_tokens;
  out.n_emitted = n_emitted;
  out.alpha_out = alpha_out;
  out.rmass_out = rmass_out;
  out.stop_out = stop_out;
  out.path_out = path_out;
  if (!L.filt) {
    float2* row_part = reinterpret_cast<float2*>(ws + L.off_row);
    float* zx = reinterpret_cast<float*>(ws + L.off_zx);
    ChunkRec* recs = reinterpret_cast<ChunkRec*>(ws + L.off_recs);
    Tie* ties = reinterpret_cast<Tie*>(ws + L.off_ties);
    if (L.small) {
      PairStat* pstat = reinterpret_cast<PairStat*>(ws + L.off_pstat);
      e = launch_verify_small(bf16, target, draft, tokens, draft_len, u, u_final, B, K, V,
                              L.nch_row, c, invT, eos_id,
                              reinterpret_cast<uint64_t*>(ws + L.off_row),
                              reinterpret_cast<uint64_t*>(ws + L.off_zx), recs, ties, pstat,
                              reinterpret_cast<uint32_t*>(ws + L.off_flags),
                              reinterpret_cast<uint32_t*>(ws + L.off_calls), out, stream);
      if (e != hipSuccess || !mark(1)) return SPECV_EHIP;
      return SPECV_OK;
    }
    e = launch_row_stats(bf16, target, draft, draft_len, tokens, B, K, V, L.nch_row, c, row_part,
                         zx, stream, 0);
    if (e != hipSuccess || !mark(1)) return SPECV_EHIP;
    e = launch_accept(bf16, false, target, draft, tokens, draft_len, u, u_final, B, K, V,
                      L.nch_row, c, invT, eos_id, row_part, zx, nullptr, out, stream);
    if (e != hipSuccess || !mark(2)) return SPECV_EHIP;
    e = launch_sample_pass(bf16, target, draft, B, K, V, L.nch_samp, invT, plan, recs, ties,
                           stream);
    if (e != hipSuccess || !mark(3)) return SPECV_EHIP;
    e = launch_sample_finish(bf16, target, draft, u_final, B, K, V, L.nch_samp, invT, plan, recs,
                             ties, out_tokens, rmass_out, stream);
    if (e != hipSuccess || !mark(4)) return SPECV_EHIP;
  } else {
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws + L.off_cand);
    int* counts = reinterpret_cast<int*>(ws + L.off_counts);
    FiltRow* frows = reinterpret_cast<FiltRow*>(ws + L.off_frows);
    Kept* kept = reinterpret_cast<Kept*>(ws + L.off_kept);
    // the candidate path has two select stages, the radix path one
    const int s0 = L.cand ? 2 : 1;
    if (L.cand)
      e = launch_filter(bf16, target, draft, draft_len, B, K, V, L.nch_filt, top_k, top_p, invT,
                        cand, counts, frows, kept, reinterpret_cast<int*>(ws + L.off_redo), stream,
                        events ? events[1] : nullptr);
    else
      e = launch_filter_rows(bf16, target, draft, draft_len, B, K, V, top_k, top_p, invT, frows,
                             kept, stream);
    if (e != hipSuccess || !mark(s0)) return SPECV_EHIP;
    e = launch_accept(bf16, true, target, draft, tokens, draft_len, u, u_final, B, K, V, 0, c,
                      invT, eos_id, nullptr, nullptr, frows, out, stream);
    if (e != hipSuccess || !mark(s0 + 1)) return SPECV_EHIP;
    // the candidate path keeps at most top_k <= 128 tokens but for ties: no
    // chunk pass for it
    e = launch_sample_list(bf16, target, draft, u_final, B, K, V, invT, plan, frows, kept,
                           L.cand ? nullptr : reinterpret_cast<double2*>(ws + L.off_cmass),
                           out_tokens, rmass_out, stream);
    if (e != hipSuccess || !mark(s0 + 2)) return SPECV_EHIP;
  }
  return SPECV_OK;
}

// Target LM head fused with verification: the layout of an unfiltered bf16
// call plus the LM head's tile statistics [B (K+1)][ntile] (float2).
struct LmLayout {
  Layout base;
  size_t off_tpart = 0, total = 0;
};

LmLayout make_lm_layout(int B, int K, int V, int top_k, float top_p) {
  LmLayout L;
  L.base = make_layout(B, K, V, true, top_k, top_p, false);
  L.off_tpart = L.base.total;
  L.total = align_up(L.off_tpart +
                     (size_t)B * (K + 1) * lm_head_tiles(V) * sizeof(float2));
  return L;
}

specv_status_t check_lm_sizes(int B, int K, int V, int D, int top_k, float top_p) {
  const specv_status_t st = check_sizes(B, K, V, SPECV_BF16, top_k, top_p);
  if (st != SPECV_OK) return st;
  if (D < 1 || D % lm_head_kblock() != 0) return SPECV_EINVAL;
  if (D > SPECV_MAX_D) return SPECV_EUNSUPPORTED;
  // the LM head's grid: vocabulary tiles x row blocks
  const size_t rows = (size_t)B * (K + 1);
  const size_t blocks = (size_t)lm_head_tiles(V) *
                        ((rows + lm_head_rows_per_block() - 1) / lm_head_rows_per_block());
  if (blocks > 0x7fffffffu || rows * (size_t)V > ((size_t)1 << 62)) return SPECV_EUNSUPPORTED;
  return SPECV_OK;
}

specv_status_t run_lm_head(const void* hidden, const void* weight, const void* draft,
                           const int32_t* tokens, const int32_t* draft_len, const float* u,
                           const float* u_final, int B, int K, int V, int D, float temperature,
                           int top_k, float top_p, int eos_id, void* target_out,
                           int32_t* out_tokens, int32_t* n_emitted, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, float* alpha_out,
                           double* rmass_out, int32_t* stop_out, int32_t* path_out) {
  specv_status_t st = check_lm_sizes(B, K, V, D, top_k, top_p);
  if (st != SPECV_OK) return st;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SPECV_EINVAL;
  if (eos_id < -1 || eos_id >= V) return SPECV_EINVAL;
  if (!hidden || !weight || !target_out || !draft_len || !u_final || !out_tokens || !n_emitted)
    return SPECV_EINVAL;
  if (K > 0 && (!draft || !tokens || !u)) return SPECV_EINVAL;
  // 16-byte loads of hidden-state rows and packed weights (D is a multiple of 64)
  if (misaligned(hidden, 16) || misaligned(weight, 16) || misaligned(target_out, 2) ||
      (draft && misaligned(draft, 2)))
    return SPECV_EINVAL;
  if (misaligned(draft_len, 4) || misaligned(u_final, 4) || misaligned(out_tokens, 4) ||
      misaligned(n_emitted, 4) || (tokens && misaligned(tokens, 4)) || (u && misaligned(u, 4)))
    return SPECV_EINVAL;
  if ((alpha_out && misaligned(alpha_out, 4)) || (rmass_out && misaligned(rmass_out, 8)) ||
      (stop_out && misaligned(stop_out, 4)) || (path_out && misaligned(path_out, 4)))
    return SPECV_EINVAL;
  const LmLayout LL = make_lm_layout(B, K, V, top_k, top_p);
  const Layout& L = LL.base;
  if (!workspace || misaligned(workspace, 16) || workspace_bytes < LL.total)
    return SPECV_EWORKSPACE;
  if (L.filt) {
    // With top-k / top-p the LM head writes the target logits, then the
    // filtered verification runs on them (its select needs the whole rows;
    // the tile statistics of the LM head's epilogue are not used).
    const float c = (float)(1.4426950408889634 / (double)temperature);
    float2* tpart = reinterpret_cast<float2*>(static_cast<char*>(workspace) + LL.off_tpart);
    if (launch_lm_head(hidden, weight, B * (K + 1), D, V, c, target_out, tpart, stream) !=
        hipSuccess)
      return SPECV_EHIP;
    return run(target_out, draft, SPECV_BF16, tokens, draft_len, u, u_final, B, K, V, temperature,
               top_k, top_p, eos_id, out_tokens, n_emitted, workspace, LL.off_tpart, stream,
               alpha_out, rmass_out, stop_out, path_out, nullptr);
  }
  char* ws = static_cast<char*>(workspace);
  Plan* plan = reinterpret_cast<Plan*>(ws + L.off_plan);
  float2* row_part = reinterpret_cast<float2*>(ws + L.off_row);
  float* zx = reinterpret_cast<float*>(ws + L.off_zx);
  ChunkRec* recs = reinterpret_cast<ChunkRec*>(ws + L.off_recs);
  Tie* ties = reinterpret_cast<Tie*>(ws + L.off_ties);
  float2* tpart = reinterpret_cast<float2*>(ws + LL.off_tpart);
  const float c = (float)(1.4426950408889634 / (double)temperature);
  const double invT = 1.0 / (double)temperature;
  AcceptOut out = {};
  out.plan = plan;
  out.out_tokens = out_tokens;
  out.n_emitted = n_emitted;
  out.alpha_out = alpha_out;
  out.rmass_out = rmass_out;
  out.stop_out = stop_out;
  out.path_out = path_out;

  // target logits and their statistics, then the draft rows' statistics; from
  // there on the call is the unfiltered verification
  hipError_t e = launch_lm_head(hidden, weight, B * (K + 1), D, V, c, target_out, tpart, stream);
  if (e == hipSuccess)
    e = launch_fold_tile_stats(tpart, target_out, tokens, B, K, V, L.nch_row, c, row_part, zx,
                               stream);
  if (e == hipSuccess && K > 0)
    e = launch_row_stats(true, target_out, draft, draft_len, tokens, B, K, V, L.nch_row, c,
                         row_part, zx, stream, K + 1);
  if (e == hipSuccess)
    e = launch_accept(true, false, target_out, draft, tokens, draft_len, u, u_final, B, K, V,
                      L.nch_row, c, invT, eos_id, row_part, zx, nullptr, out, stream);
  if (e == hipSuccess)
    e = launch_sample_pass(true, target_out, draft, B, K, V, L.nch_samp, invT, plan, recs, ties,
                           stream);
  if (e == hipSuccess)
    e = launch_sample_finish(true, target_out, draft, u_final, B, K, V, L.nch_samp, invT, plan,
                             recs, ties, out_tokens, rmass_out, stream);
  return e == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

// Scratch of the allocation-free entry point: one fixed array in device
// memory, held by every GPU the library runs on until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SPECV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on `device` (the current device), or null on error.
void* scratch_on(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[device].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[device].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[device].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace specv

extern "C" {

size_t specv_workspace_bytes(int B, int K, int V, specv_dtype_t dtype, int top_k, float top_p) {
  if (specv::check_sizes(B, K, V, dtype, top_k, top_p) != SPECV_OK) return 0;
  return specv::make_layout(B, K, V, dtype == SPECV_BF16, top_k, top_p).total;
}

specv_status_t specv_verify(const void* target_logits, const void* draft_logits,
                            specv_dtype_t dtype, const int32_t* draft_tokens,
                            const int32_t* draft_len, const float* u, const float* u_final,
                            int B, int K, int V, float temperature, int top_k, float top_p,
                            int eos_id, int32_t* out_tokens, int32_t* n_emitted, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return specv::run(target_logits, draft_logits, dtype, draft_tokens, draft_len, u, u_final, B,
                    K, V, temperature, top_k, top_p, eos_id, out_tokens, n_emitted, workspace,
                    workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr, nullptr);
}

specv_status_t specv_verify_noalloc(const void* target_logits, const void* draft_logits,
                                    specv_dtype_t dtype, const int32_t* draft_tokens,
                                    const int32_t* draft_len, const float* u, const float* u_final,
                                    int B, int K, int V, float temperature, int top_k,
                                    float top_p, int eos_id, int32_t* out_tokens,
                                    int32_t* n_emitted, hipStream_t stream) {
  using namespace specv;
  // Sizes first, on the host: too large for the fixed scratch is an error
  // before any device is touched.
  const specv_status_t st = check_sizes(B, K, V, dtype, top_k, top_p);
  if (st != SPECV_OK) return st;
  if (make_layout(B, K, V, dtype == SPECV_BF16, top_k, top_p).total > SPECV_NOALLOC_SCRATCH_BYTES)
    return SPECV_ESCRATCH;
  // The scratch of the device the stream belongs to, looked up with that
  // device current.
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SPECV_EHIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return SPECV_EHIP;
  void* ws = nullptr;
  if (dev == cur) {
    ws = scratch_on(dev);
  } else {
    if (hipSetDevice(dev) != hipSuccess) return SPECV_EHIP;
    ws = scratch_on(dev);
    if (hipSetDevice(cur) != hipSuccess) return SPECV_EHIP;
  }
  if (!ws) return SPECV_EHIP;
  return run(target_logits, draft_logits, dtype, draft_tokens, draft_len, u, u_final, B, K, V,
             temperature, top_k, top_p, eos_id, out_tokens, n_emitted, ws,
             SPECV_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, nullptr, nullptr, nullptr);
}

specv_status_t specv_verify_debug(const void* target_logits, const void* draft_logits,
                                  specv_dtype_t dtype, const int32_t* draft_tokens,
                                  const int32_t* draft_len, const float* u,
                                  const float* u_final, int B, int K, int V, float temperature,
                                  int top_k, float top_p, int eos_id, int32_t* out_tokens,
                                  int32_t* n_emitted, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, float* accept_prob, double* residual_mass,
                                  int32_t* stop_pos, int32_t* path) {
  return specv::run(target_logits, draft_logits, dtype, draft_tokens, draft_len, u, u_final, B,
                    K, V, temperature, top_k, top_p, eos_id, out_tokens, n_emitted, workspace,
                    workspace_bytes, stream, accept_prob, residual_mass, stop_pos, path,
                    nullptr);
}

specv_status_t specv_verify_timed(const void* target_logits, const void* draft_logits,
                                  specv_dtype_t dtype, const int32_t* draft_tokens,
                                  const int32_t* draft_len, const float* u,
                                  const float* u_final, int B, int K, int V, float temperature,
                                  int top_k, float top_p, int eos_id, int32_t* out_tokens,
                                  int32_t* n_emitted, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, hipEvent_t* events) {
  if (!events) return SPECV_EINVAL;
  const int nst = specv::kNumStages[specv::path_kind(B, K, V, top_k, top_p)];
  for (int i = 0; i <= nst; ++i)
    if (!events[i]) return SPECV_EINVAL;
  return specv::run(target_logits, draft_logits, dtype, draft_tokens, draft_len, u, u_final, B,
                    K, V, temperature, top_k, top_p, eos_id, out_tokens, n_emitted, workspace,
                    workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr, events);
}

int specv_num_stages(int kind) {
  return (kind >= 0 && kind < specv::kNumPaths) ? specv::kNumStages[kind] : 0;
}

int specv_path_kind(int B, int K, int V, int top_k, float top_p) {
  return specv::path_kind(B, K, V, top_k, top_p);
}

int specv_selftest_set_small_poll_limit(int limit) { return specv::set_small_poll_limit(limit); }

long long specv_set_small_batch_limit(long long limit) {
  return specv::g_small_limit.exchange(limit < 0 ? 0 : limit);
}

specv_status_t specv_bench_row_stats(const void* const* targets, const void* const* drafts,
                                     const int32_t* const* draft_tokens,
                                     const int32_t* const* draft_lens, int nsets,
                                     specv_dtype_t dtype, int B, int K, int V, float temperature,
                                     void* workspace, size_t workspace_bytes, int reps,
                                     hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  using namespace specv;
  if (check_sizes(B, K, V, dtype, 0, 1.0f) != SPECV_OK) return SPECV_EINVAL;
  if (!targets || !drafts || !draft_tokens || !draft_lens || nsets < 1 || reps < 1 || !start ||
      !stop)
    return SPECV_EINVAL;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SPECV_EINVAL;
  const size_t esz = dtype == SPECV_BF16 ? 2 : 4;
  for (int i = 0; i < nsets; ++i) {
    if (!targets[i] || !draft_lens[i] || misaligned(targets[i], esz) ||
        misaligned(draft_lens[i], 4))
      return SPECV_EINVAL;
    if (K > 0 && (!drafts[i] || !draft_tokens[i] || misaligned(drafts[i], esz) ||
                  misaligned(draft_tokens[i], 4)))
      return SPECV_EINVAL;
  }
  const bool bf16 = dtype == SPECV_BF16;
  const Layout L = make_layout(B, K, V, bf16, 0, 1.0f);
  if (!workspace || misaligned(workspace, 16) || workspace_bytes < L.total) return SPECV_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float2* row_part = reinterpret_cast<float2*>(ws + L.off_row);
  float* zx = reinterpret_cast<float*>(ws + L.off_zx);
  const float c = (float)(1.4426950408889634 / (double)temperature);
  if (hipEventRecord(start, stream) != hipSuccess) return SPECV_EHIP;
  for (int r = 0; r < reps; ++r) {
    const int i = r % nsets;
    if (launch_row_stats(bf16, targets[i], drafts[i], draft_lens[i], draft_tokens[i], B, K, V,
                         L.nch_row, c, row_part, zx, stream) != hipSuccess)
      return SPECV_EHIP;
  }
  return hipEventRecord(stop, stream) == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

size_t specv_lm_head_packed_weight_bytes(int V, int D) {
  if (V < 1 || V > SPECV_MAX_V || D < 1 || D % specv::lm_head_kblock() != 0 || D > SPECV_MAX_D)
    return 0;
  return specv::lm_head_packed_elems(V, D) * sizeof(uint16_t);
}

specv_status_t specv_lm_head_pack_weight(const void* lm_head_weight, void* packed_weight, int V,
                                         int D, hipStream_t stream) {
  using namespace specv;
  if (V < 1 || V > SPECV_MAX_V || D < 1 || D % lm_head_kblock() != 0 || D > SPECV_MAX_D)
    return SPECV_EINVAL;
  if (!lm_head_weight || !packed_weight || misaligned(lm_head_weight, 16) ||
      misaligned(packed_weight, 16))
    return SPECV_EINVAL;
  // the packed copy must not overlap the source
  const char* a = static_cast<const char*>(lm_head_weight);
  const char* p = static_cast<const char*>(packed_weight);
  const size_t na = (size_t)V * D * sizeof(uint16_t);
  const size_t np = lm_head_packed_elems(V, D) * sizeof(uint16_t);
  if (a < p + np && p < a + na) return SPECV_EINVAL;
  return launch_lm_head_pack(lm_head_weight, packed_weight, V, D, stream) == hipSuccess
             ? SPECV_OK
             : SPECV_EHIP;
}

size_t specv_lm_head_workspace_bytes(int B, int K, int V, int D, int top_k, float top_p) {
  if (specv::check_lm_sizes(B, K, V, D, top_k, top_p) != SPECV_OK) return 0;
  return specv::make_lm_layout(B, K, V, top_k, top_p).total;
}

specv_status_t specv_verify_lm_head(const void* hidden, const void* packed_weight,
                                    const void* draft_logits, const int32_t* draft_tokens,
                                    const int32_t* draft_len, const float* u,
                                    const float* u_final, int B, int K, int V, int D,
                                    float temperature, int top_k, float top_p, int eos_id,
                                    void* target_logits, int32_t* out_tokens,
                                    int32_t* n_emitted, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream, float* accept_prob,
                                    double* residual_mass, int32_t* stop_pos, int32_t* path) {
  return specv::run_lm_head(hidden, packed_weight, draft_logits, draft_tokens, draft_len, u,
                            u_final, B, K, V, D, temperature, top_k, top_p, eos_id,
                            target_logits, out_tokens, n_emitted, workspace, workspace_bytes,
                            stream, accept_prob, residual_mass, stop_pos, path);
}

specv_status_t specv_bench_lm_head(const void* hidden, const void* packed_weight, int M, int D,
                                   int V, float temperature, void* logits, void* workspace,
                                   size_t workspace_bytes, int reps, hipStream_t stream,
                                   hipEvent_t start, hipEvent_t stop) {
  using namespace specv;
  if (M < 1 || V < 1 || V > SPECV_MAX_V || D < 1 || D % lm_head_kblock() != 0 ||
      D > SPECV_MAX_D || reps < 1 || !start || !stop)
    return SPECV_EINVAL;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SPECV_EINVAL;
  if (!hidden || !packed_weight || !logits || misaligned(hidden, 16) ||
      misaligned(packed_weight, 16) || misaligned(logits, 2))
    return SPECV_EINVAL;
  const size_t need = (size_t)M * lm_head_tiles(V) * sizeof(float2);
  if (!workspace || misaligned(workspace, 16) || workspace_bytes < need) return SPECV_EWORKSPACE;
  const float c = (float)(1.4426950408889634 / (double)temperature);
  if (hipEventRecord(start, stream) != hipSuccess) return SPECV_EHIP;
  for (int i = 0; i < reps; ++i)
    if (launch_lm_head(hidden, packed_weight, M, D, V, c, logits,
                       static_cast<float2*>(workspace), stream) != hipSuccess)
      return SPECV_EHIP;
  return hipEventRecord(stop, stream) == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

specv_status_t specv_sample(const void* logits, specv_dtype_t dtype, const float* u, int R, int V,
                            float temperature, int top_k, float top_p, int32_t* out_tokens,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return specv::run(logits, nullptr, dtype, nullptr, nullptr, nullptr, u, R, 0, V, temperature,
                    top_k, top_p, -1, out_tokens, nullptr, workspace, workspace_bytes, stream,
                    nullptr, nullptr, nullptr, nullptr, nullptr, true);
}

specv_status_t specv_acceptance_rates(const void* target_logits, const void* draft_logits,
                                      specv_dtype_t dtype, const int32_t* draft_len, int B,
                                      int K, int V, float temperature, int top_k, float top_p,
                                      float* beta, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  using namespace specv;
  specv_status_t st = check_sizes(B, K, V, dtype, top_k, top_p);
  if (st != SPECV_OK) return st;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SPECV_EINVAL;
  const size_t esz = dtype == SPECV_BF16 ? 2 : 4;
  if (!target_logits || !draft_len || !beta || (K > 0 && !draft_logits)) return SPECV_EINVAL;
  if (misaligned(target_logits, esz) || (draft_logits && misaligned(draft_logits, esz)) ||
      misaligned(draft_len, 4) || misaligned(beta, 4))
    return SPECV_EINVAL;
  const bool bf16 = dtype == SPECV_BF16;
  const Layout L = make_layout(B, K, V, bf16, top_k, top_p);
  if (!workspace || misaligned(workspace, 16) || workspace_bytes < L.total) return SPECV_EWORKSPACE;
  if (K == 0) return SPECV_OK;
  char* ws = static_cast<char*>(workspace);
  const float c = (float)(1.4426950408889634 / (double)temperature);
  const double invT = 1.0 / (double)temperature;
  hipError_t e;
  if (!L.filt) {
    float2* row_part = reinterpret_cast<float2*>(ws + L.off_row);
    // the rows of drafted positions only, through the cache: beta_pass reads
    // them again right after
    e = launch_row_stats(bf16, target_logits, draft_logits, draft_len, nullptr, B, K, V,
                         L.nch_row, c, row_part, nullptr, stream, 0, true, true);
    if (e == hipSuccess)
      e = launch_beta(bf16, false, target_logits, draft_logits, draft_len, B, K, V, L.nch_row,
                      c, invT, row_part, nullptr, nullptr,
                      reinterpret_cast<float*>(ws + L.off_beta), beta, stream);
  } else {
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws + L.off_cand);
    int* counts = reinterpret_cast<int*>(ws + L.off_counts);
    FiltRow* frows = reinterpret_cast<FiltRow*>(ws + L.off_frows);
    Kept* kept = reinterpret_cast<Kept*>(ws + L.off_kept);
    if (L.cand)
      e = launch_filter(bf16, target_logits, draft_logits, draft_len, B, K, V, L.nch_filt, top_k,
                        top_p, invT, cand, counts, frows, kept,
                        reinterpret_cast<int*>(ws + L.off_redo), stream, nullptr);
    else
      e = launch_filter_rows(bf16, target_logits, draft_logits, draft_len, B, K, V, top_k, top_p,
                             invT, frows, kept, stream);
    if (e == hipSuccess)
      e = launch_beta(bf16, true, target_logits, draft_logits, draft_len, B, K, V, 0, c, invT,
                      nullptr, frows, kept, nullptr, beta, stream);
  }
  return e == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

specv_status_t specv_round_stats(const int32_t* draft_tokens, const int32_t* draft_len,
                                 const int32_t* out_tokens, const int32_t* n_emitted,
                                 const float* beta, int B, int K, int32_t* accepted,
                                 float* expected, int64_t* totals, hipStream_t stream) {
  using namespace specv;
  if (B < 1 || K < 0 || K > SPECV_MAX_K) return SPECV_EINVAL;
  if ((K > 0 && !draft_tokens) || !draft_len || !out_tokens || !n_emitted) return SPECV_EINVAL;
  if (expected && !beta) return SPECV_EINVAL;
  if ((draft_tokens && misaligned(draft_tokens, 4)) || misaligned(draft_len, 4) ||
      misaligned(out_tokens, 4) || misaligned(n_emitted, 4) || (beta && misaligned(beta, 4)) ||
      (accepted && misaligned(accepted, 4)) || (expected && misaligned(expected, 4)) ||
      (totals && misaligned(totals, 8)))
    return SPECV_EINVAL;
  const hipError_t e =
      launch_round_stats(draft_tokens, draft_len, out_tokens, n_emitted, beta, B, K, accepted,
                         expected, reinterpret_cast<long long*>(totals), stream);
  return e == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

size_t specv_monitor_state_bytes(int B, int window) {
  if (B < 1 || window < 1 || window > SPECV_MAX_WINDOW) return 0;
  return specv::monitor_state_bytes(B, window);
}

specv_status_t specv_monitor_reset(void* state, int B, int window, hipStream_t stream) {
  using namespace specv;
  if (B < 1 || window < 1 || window > SPECV_MAX_WINDOW) return SPECV_EINVAL;
  if (!state || misaligned(state, 16)) return SPECV_EINVAL;
  return launch_monitor_reset(state, B, window, stream) == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

specv_status_t specv_monitor_update(const int32_t* draft_tokens, const int32_t* draft_len,
                                    const int32_t* out_tokens, const int32_t* n_emitted, int B,
                                    int K, int max_k, int window, void* state,
                                    int32_t* next_draft_len, double* rate, hipStream_t stream) {
  using namespace specv;
  if (B < 1 || K < 0 || K > SPECV_MAX_K || max_k < 1 || max_k > SPECV_MAX_K) return SPECV_EINVAL;
  if (window < 1 || window > SPECV_MAX_WINDOW) return SPECV_EINVAL;
  if ((K > 0 && !draft_tokens) || !draft_len || !out_tokens || !n_emitted || !state ||
      !next_draft_len)
    return SPECV_EINVAL;
  if ((draft_tokens && misaligned(draft_tokens, 4)) || misaligned(draft_len, 4) ||
      misaligned(out_tokens, 4) || misaligned(n_emitted, 4) || misaligned(state, 16) ||
      misaligned(next_draft_len, 4) || (rate && misaligned(rate, 8)))
    return SPECV_EINVAL;
  const hipError_t e = launch_monitor_update(draft_tokens, draft_len, out_tokens, n_emitted, B, K,
                                             max_k, window, state, next_draft_len, rate, stream);
  return e == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

specv_status_t specv_selftest_exp64(const double* x, double* y, int n, hipStream_t stream) {
  if (n < 0 || (n > 0 && (!x || !y))) return SPECV_EINVAL;
  return specv::launch_exp64_selftest(x, y, n, stream) == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

const char* specv_stage_name(int kind, int i) {
  if (kind < 0 || kind >= specv::kNumPaths) return nullptr;
  return (i >= 0 && i < specv::kNumStages[kind]) ? specv::kStageNames[kind][i] : nullptr;
}

const char* specv_status_string(specv_status_t status) {
  switch (status) {
    case SPECV_OK: return "ok";
    case SPECV_EINVAL: return "invalid argument";
    case SPECV_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SPECV_EHIP: return "HIP launch failed";
    case SPECV_EUNSUPPORTED: return "unsupported parameter combination";
    case SPECV_ESCRATCH:
      return "sizes need more scratch than the allocation-free call's fixed array holds";
  }
  return "unknown status";
}

int specv_version(void) { return 103; }

}  // extern "C"
