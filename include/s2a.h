/*
 * s2a.h -- C ABI of libs2a.so: shifted short attention (S2-Attn) and bounded-history
 * attention (HGA) for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device, owned by the
 *    caller (the one exception, the host-tier history of hga_detach_segment and
 *    hga_stage_selected, is pinned host memory).  The library never allocates, frees or
 *    keeps a pointer past the call.  Its only state is a per-device cache of the
 *    compute-unit count and of the address of the static scratch array of
 *    s2attn_bwd_noalloc (both written once, thread-safe); calls that take their workspace
 *    from the caller on different streams are independent.
 *  - bf16 tensors are passed as raw 16-bit storage (bfloat16 bit patterns).
 *  - Layouts are row-major with the head dimension d contiguous:
 *        queries / outputs / output-gradients   [B, L, H,   d]
 *        keys / values                          [B, L, Hkv, d]
 *        log-sum-exp                            [B, H, L]   float32, natural log
 *    Every tensor pointer must be 16-byte aligned.
 *  - Outputs are overwritten, never accumulated into.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Launches are asynchronous;
 *    nothing is launched unless every argument check passes.  A status other than
 *    S2A_OK means nothing was launched, except S2A_ERR_HIP, which reports a launch
 *    error returned by the runtime.  Faults inside a kernel surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - q head h reads kv head floor(h * Hkv / H) (grouped-query attention); gradients of a
 *    kv head are the sum over its q heads.
 *  - Supported head dims: d in {64, 128}; other values return S2A_ERR_UNSUPPORTED.
 */
#ifndef S2A_H
#define S2A_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  S2A_OK = 0,
  S2A_ERR_INVALID_ARG = 1,  /* a null/misaligned pointer, a non-positive or inconsistent size */
  S2A_ERR_UNSUPPORTED = 2,  /* a valid request this build does not implement (d, tile rules) */
  S2A_ERR_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_bytes() */
  S2A_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} s2a_status;

/* Human-readable name of a status code (static storage). */
const char* s2a_status_string(int status);

/* ------------------------------------------------------------------------------------
 * Shifted short attention, forward.
 *
 * LongLoRA ("LongLoRA: Efficient Fine-tuning of Long-Context Large Language Models",
 * English abstract) and the LongQLoRA post (section 03, Shift Short Attention
 * paragraph): tokens are split into groups of G and attention runs causally inside each
 * group; to let information cross group borders, half of the heads see the sequence
 * shifted by half a group.  Here: when `shift` != 0 and N/G >= 2, q heads [H/2, H) see
 * token t at rolled position p(t) = (t - G/2) mod N, in group floor(p/G), and key u is
 * visible to query t iff both sit in the same rolled group and p(u) <= p(t) (causal in
 * rolled order, i.e. roll - attend - roll back).  Other heads (and every head when
 * G == N) use p(t) = t.  The roll is indexed, never materialised; O is in token order.
 *
 *   q [B,N,H,d], k/v [B,N,Hkv,d] bf16 (in);  o [B,N,H,d] bf16 (out);
 *   lse [B,H,N] float32 (out) = log sum_u exp(scale * q_t . k_u) over visible u.
 *
 * Checks: B,N,H,Hkv,G > 0; H % Hkv == 0; N % G == 0; G % 64 == 0 (else UNSUPPORTED);
 * when shifting: (G/2) % 64 == 0 (else UNSUPPORTED) and Hkv even (so shifted q heads map
 * to shifted kv heads; else INVALID_ARG).  scale must be finite and > 0.
 * ------------------------------------------------------------------------------------ */
int s2attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int N, int H, int Hkv, int d, int G, int shift, float scale,
               void* stream);

/* Workspace bytes s2attn_bwd needs for these sizes: two float32 [B, H, N] row statistics,
 * D = rowsum(dO * O) and LSE * log2(e). */
size_t s2attn_bwd_workspace_bytes(int B, int N, int H, int Hkv, int d);

/* Workspace bytes that let s2attn_bwd keep dS (LongLoRA S2-Attn backward, same
 * definitions as below) between its key-major and query-major halves: the row statistics,
 * padded to 256 bytes, then bf16 dS = P * (dP - D) of every lower-triangle 64 x 64 tile
 * of every (batch, head, group).  Given a workspace at least this large, s2attn_bwd
 * computes dQ = scale dS K from the stored tiles instead of recomputing S and dP; results
 * agree with the smaller workspace's to bf16 rounding of dS, and are deterministic.
 * 2 bytes per lower-triangle element: 553 MB at B=1, N=8192, H=32, G=2048; 8.7 GB at
 * N=32768, G=8192.  0 for invalid sizes (B, N, H not positive, or G not a positive
 * multiple of 64 dividing N). */
size_t s2attn_bwd_workspace_bytes_dsq(int B, int N, int H, int Hkv, int d, int G);

/* ------------------------------------------------------------------------------------
 * Shifted short attention, backward (same mask as s2attn_fwd; same pages).
 *
 * With P = exp(scale * q.k - lse) on the mask: dV = P^T dO, dP = dO V^T,
 * D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *   in:  q, k, v, o (bf16), lse (float32, from s2attn_fwd), dout [B,N,H,d] bf16
 *   out: dq [B,N,H,d], dk/dv [B,N,Hkv,d] bf16
 *   workspace: device scratch of at least s2attn_bwd_workspace_bytes(...) bytes, owned
 *   by the caller, contents undefined on entry and on exit.  With at least
 *   s2attn_bwd_workspace_bytes_dsq(...) bytes, dQ is computed from stored dS tiles.
 * Deterministic: no atomics; the same inputs give the same bits.
 * ------------------------------------------------------------------------------------ */
int s2attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes,
               int B, int N, int H, int Hkv, int d, int G, int shift, float scale,
               void* stream);

/* ------------------------------------------------------------------------------------
 * s2attn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight training loops, harnesses that forbid
 * hipMalloc).  Same arguments (minus the workspace), checks, results and bits as
 * s2attn_bwd with a workspace of s2attn_bwd_workspace_bytes(...) bytes (dQ recomputed,
 * no dS tiles).  The row statistics go to a static device array of
 * S2A_NOALLOC_SCRATCH_BYTES bytes inside the library: one copy per GPU, held until the
 * process ends; its address is looked up once per device with hipGetSymbolAddress.  The
 * call allocates and frees nothing.
 * Limit: s2attn_bwd_workspace_bytes(B, N, H, Hkv, d) <= S2A_NOALLOC_SCRATCH_BYTES, i.e.
 * B * H * N <= 1048576 rows (e.g. 32 heads x 32768 tokens); larger sizes return
 * S2A_ERR_WORKSPACE and launch nothing.  S2A_ERR_HIP if the runtime cannot report the
 * array's address.
 * Concurrency: every call on one GPU uses that GPU's single array, so calls that can
 * overlap on one GPU (different streams, or different host threads without ordering)
 * race; serialise them.  Nothing in the array needs clearing: each call writes every
 * value it reads before reading it.
 * ------------------------------------------------------------------------------------ */
#define S2A_NOALLOC_SCRATCH_BYTES (8u << 20)

int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv,
                       int B, int N, int H, int Hkv, int d, int G, int shift, float scale,
                       void* stream);

/* The stages of s2attn_bwd on `stream`, for callers that want to time them or overlap
 * dQ and dK/dV on separate streams.  Same arguments, checks and layouts as s2attn_bwd;
 * the workspace must be the one the statistics were written to.
 *   prep:    D = rowsum(dO * O) and LSE * log2(e) into the workspace
 *   dq:      dQ (query-major kernel); reads the workspace
 *   dkdv:    dK and dV (key-major kernels, grouped-query sum in registers); reads the
 *            workspace
 *   dq_prep: prep and dq in one kernel (what s2attn_bwd runs): the dQ kernel computes
 *            the statistics of the rows it owns and writes them to the workspace, so
 *            dkdv must be ordered after it.
 * With a workspace of s2attn_bwd_workspace_bytes(...) bytes, s2attn_bwd is dq_prep
 * followed by dkdv; to run dq and dkdv concurrently, run prep first and then both (they
 * only read the workspace).  With one of s2attn_bwd_workspace_bytes_dsq(...) bytes, dkdv
 * also stores the dS tiles into it and dq forms dQ from them, so dq must follow dkdv
 * (s2attn_bwd is then prep, dkdv, dq); dq_prep still recomputes. */
int s2attn_bwd_prep(const void* o, const float* lse, const void* dout, void* workspace, size_t workspace_bytes,
                    int B, int N, int H, int Hkv, int d, int G, int shift, float scale, void* stream);
int s2attn_bwd_dq_prep(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* workspace, size_t workspace_bytes, int B, int N, int H,
                       int Hkv, int d, int G, int shift, float scale, void* stream);
int s2attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, const void* workspace,
                  size_t workspace_bytes, int B, int N, int H, int Hkv, int d, int G, int shift, float scale,
                  void* stream);
int s2attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                    const void* workspace, size_t workspace_bytes, int B, int N, int H, int Hkv, int d, int G,
                    int shift, float scale, void* stream);

/* ------------------------------------------------------------------------------------
 * HGA chunk summaries.
 *
 * "Long-Context Fine-Tuning with Limited VRAM" (BMW Group, English abstract): resident
 * chunk summaries are kept for the detached history.  Here a summary is the mean key of
 * a chunk, per kv head:  summ[b, c, j, :] = (1/chunk) sum_{i<chunk} k_hist[b, c*chunk+i, j, :].
 *   k_hist: bf16, element (b, t, j, e) at k_hist[b*hist_bstride + (t*Hkv + j)*d + e]
 *   summ:   float32, element (b, c, j, e) at summ[b*summ_bstride + (c*Hkv + j)*d + e]
 * Strides are in elements, so the history may be a prefix of a longer buffer and new
 * summaries can be appended by offsetting `summ` by c0*Hkv*d.
 * Checks: T % chunk == 0 (T == 0 is a no-op), chunk % 64 == 0, strides large enough.
 * ------------------------------------------------------------------------------------ */
int hga_summarize(const void* k_hist, long long hist_bstride, float* summ, long long summ_bstride,
                  int B, int T, int Hkv, int d, int chunk, void* stream);

/* ------------------------------------------------------------------------------------
 * HGA history append (same page: once a segment is done its keys and values leave the
 * autograd graph and join the history, and the summary table grows by its chunks).
 * Copies keys and values of S segment tokens into history rows [T, T + S) and writes the
 * summaries of the new chunks, in one pass:
 *   k_hist[b, T + t, j, :] = k_seg[b, t, j, :],  v_hist likewise        (bit-exact copy)
 *   summ[b, T/chunk + c, j, :] = (1/chunk) sum_{i<chunk} k_seg[b, c*chunk + i, j, :]
 *   k_seg/v_seg: bf16, element (b, t, j, e) at k_seg[b*seg_bstride + (t*Hkv + j)*d + e]
 *   k_hist/v_hist: bf16 with hist_bstride, room for T + S tokens; summ as in hga_summarize,
 *   room for (T + S)/chunk chunks.  Rows [0, T) of the history and summaries [0, T/chunk)
 *   are left untouched.  The segment and the destination rows must not overlap unless
 *   they coincide (an in-place append only writes the summaries' values again).
 * Checks: S % chunk == 0 and T % chunk == 0 (S == 0 is a no-op), chunk % 64 == 0,
 * strides large enough, (T + S) * Hkv * d < 2^31.
 * ------------------------------------------------------------------------------------ */
int hga_append_history(const void* k_seg, const void* v_seg, long long seg_bstride, void* k_hist, void* v_hist,
                       long long hist_bstride, float* summ, long long summ_bstride, int B, int S, int Hkv, int d,
                       int T, int chunk, void* stream);

/* ------------------------------------------------------------------------------------
 * HGA per-query-block chunk selection (same page: every query block gets a capped
 * selection of history chunks).  Score of chunk c for (b, q head h, block j):
 *   qbar = mean of the block's `qblock` queries of head h (float32),
 *   score = qbar . summ[b, c, kv(h), :]        (no 1/sqrt(d) factor)
 * The k_eff = min(topk, C) highest scores are kept, ties going to the lower chunk index;
 * idx[b, h, j, :] lists them ascending, followed by -1 padding.  C == 0 gives all -1.
 *   q [B,S,H,d] bf16;  summ as in hga_summarize;  idx [B, H, S/qblock, topk] int32 (out)
 * Checks: S % qblock == 0, qblock == 64, 1 <= topk <= 64, C >= 0.
 * ------------------------------------------------------------------------------------ */
int hga_select_topk(const void* q, const float* summ, long long summ_bstride, int32_t* idx,
                    int B, int S, int H, int Hkv, int d, int C, int qblock, int topk,
                    void* stream);

/* ------------------------------------------------------------------------------------
 * HGA forward (same page: each query block attends to the full tokens of its selected
 * history chunks plus its own segment).  Query t (segment position) of block j = t / qblock
 * attends, under ONE softmax with logit scale `scale`, to
 *   (i)  active keys u <= t, and
 *   (ii) every token of each chunk listed in idx[b, h, j, :] (entries >= 0; -1 = none).
 *   q [B,S,H,d] bf16; k_act/v_act bf16 with element (b,t,j,e) at
 *   k_act[b*act_bstride + (t*Hkv+j)*d + e]; k_hist/v_hist likewise with hist_bstride
 *   (T tokens); idx [B,H,S/qblock,topk] int32, each valid entry < T/chunk.
 *   out: o [B,S,H,d] bf16, lse [B,H,S] float32.
 * Checks: S % qblock == 0, qblock == 64, T % chunk == 0, chunk % 64 == 0,
 * 1 <= topk <= 64.  Index values are not range-checked on the host (they live on the
 * device); out-of-range entries are skipped by the kernel.
 * ------------------------------------------------------------------------------------ */
int hga_fwd(const void* q, const void* k_act, const void* v_act, long long act_bstride,
            const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
            void* o, float* lse,
            int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk, float scale,
            void* stream);

/* Workspace bytes hga_bwd_active needs for these sizes (0 for sizes it rejects): two
 * float32 [B, H, S] row statistics (D = rowsum(dO * O) and LSE * log2(e)), plus, when the
 * segment alone would leave most compute units idle (B * Hkv * ceil(S / 128) < 256), the
 * float32 partial sums of the split dK/dV work. */
size_t hga_bwd_workspace_bytes(int B, int S, int H, int Hkv, int d);

/* Workspace bytes with which hga_bwd_active (and _shared) stores dS (0 for sizes they
 * reject): hga_bwd_workspace_bytes(...) rounded up to 256, plus the bf16 dS tiles of every
 * (batch, q head)'s causal local part, B * H * t (t + 1) / 2 tiles of 64 x 64 with t = S / 64
 * (138 MB at B = 1, S = 2048, H = 32).  Given at least this much, the backward computes the
 * row statistics first, the dK/dV kernel stores dS of the local keys, and the dQ kernel takes
 * the local part of dQ = scale dS K from those tiles instead of recomputing S and dP there
 * (the history part is recomputed either way).  Given less, it recomputes.  Both give dQ, dK
 * and dV to the same tolerance; the bits differ (the row statistics are summed in another
 * order). */
size_t hga_bwd_workspace_bytes_dsq(int B, int S, int H, int Hkv, int d);

/* ------------------------------------------------------------------------------------
 * HGA backward, active segment only (same page: gradients reach the current segment
 * alone; the history's keys and values are cut off from the graph).  Same key sets as
 * hga_fwd; the selection is held fixed.  dq covers the local and the history keys;
 * dk_act/dv_act come from the local keys only; the history receives no gradient.
 *   in: hga_fwd's inputs, o and lse from hga_fwd, dout [B,S,H,d] bf16
 *   out: dq [B,S,H,d], dk_act/dv_act [B,S,Hkv,d] (contiguous) bf16
 *   workspace: at least hga_bwd_workspace_bytes(...) bytes (hga_bwd_workspace_bytes_dsq(...)
 *   for the stored-dS path), owned by the caller, contents undefined on entry and on exit.
 * Deterministic: no atomics; split dK/dV partial sums are added in a fixed order.
 * ------------------------------------------------------------------------------------ */
int hga_bwd_active(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                   const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                   const void* o, const float* lse, const void* dout,
                   void* dq, void* dk_act, void* dv_act,
                   void* workspace, size_t workspace_bytes,
                   int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk, float scale,
                   void* stream);

/* ------------------------------------------------------------------------------------
 * HGA with one chunk selection per kv head, shared by its H/Hkv q heads (a reading of the
 * same page, which caps the chunks per query block but does not say whether the q heads of a
 * grouped-query-attention group choose together).  Score of chunk c for (b, kv head g,
 * block j): (sum over the q heads h of g of qbar_h) . summ[b, c, g, :], i.e. the sum of
 * the heads' hga_select_topk scores.  Same top-k, tie and padding rules as hga_select_topk.
 *   idx [B, Hkv, S/qblock, topk] int32 (out)
 * hga_fwd_shared and hga_bwd_active_shared take that idx: every q head h attends to the
 * chunks listed for its kv head h / (H/Hkv); everything else is as in hga_fwd and
 * hga_bwd_active (same arguments, checks, workspace and outputs).  With H == Hkv the two
 * forms coincide.
 * ------------------------------------------------------------------------------------ */
int hga_select_topk_shared(const void* q, const float* summ, long long summ_bstride, int32_t* idx,
                           int B, int S, int H, int Hkv, int d, int C, int qblock, int topk,
                           void* stream);
int hga_fwd_shared(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                   const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                   void* o, float* lse,
                   int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk, float scale,
                   void* stream);
int hga_bwd_active_shared(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                          const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
                          const void* o, const float* lse, const void* dout,
                          void* dq, void* dk_act, void* dv_act,
                          void* workspace, size_t workspace_bytes,
                          int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk,
                          float scale, void* stream);

/* ------------------------------------------------------------------------------------
 * HGA forward that selects its own chunk lists (one per kv head and query block, as
 * hga_select_topk_shared) and attends to them in the same launch: selection and
 * attention of the same page (each query block scores the history chunks against their
 * summaries, keeps a capped set and attends to all of its tokens).  Results equal
 * hga_select_topk_shared followed by hga_fwd_shared, bit for bit; the lists are also
 * written to idx for the backward (hga_bwd_active_shared).
 *   inputs as hga_fwd_shared, plus summ (as in hga_select_topk, C = T/chunk chunks; may be
 *   NULL when T == 0) with its batch stride;
 *   out: idx [B, Hkv, S/qblock, topk] int32, o [B,S,H,d] bf16, lse [B,H,S] float32.
 * Kv heads with four q heads run one launch (each workgroup scores its block's chunks
 * before attending); other group sizes run the two launches.
 * Checks: those of hga_fwd_shared, plus summ non-null when T > 0 and summ_bstride large
 * enough.
 * ------------------------------------------------------------------------------------ */
int hga_fwd_select_shared(const void* q, const void* k_act, const void* v_act, long long act_bstride,
                          const void* k_hist, const void* v_hist, long long hist_bstride,
                          const float* summ, long long summ_bstride, int32_t* idx, void* o, float* lse,
                          int B, int S, int H, int Hkv, int d, int T, int chunk, int qblock, int topk,
                          float scale, void* stream);

/* ------------------------------------------------------------------------------------
 * HGA host-tier history (same page: the older keys and values are moved out of GPU memory
 * into host RAM, and each query block needs only the few whole chunks selected for it).
 * The history rows live in PINNED host memory (hipHostMalloc, or an allocator built on
 * it, such as torch's pin_memory) that the GPU reads and writes over the host link; the
 * chunk summaries stay in device memory.  Pageable host memory and device memory are
 * rejected with S2A_ERR_INVALID_ARG for the host-tier arguments.
 *
 * hga_detach_segment: hga_append_history with the history rows in host memory.  The
 *   segment K/V and summ are device memory; k_host/v_host [B, >= T+S, Hkv, d] bf16 with
 *   batch stride host_bstride receive rows [T, T + S).  Same checks as hga_append_history.
 *
 * hga_stage_selected: gathers the chunks a set of chunk lists names into a device staging
 *   history and rewrites the lists to it, so that the attention entry points run on the
 *   staging history with the same results, bit for bit, as on the full history:
 *     idx [B, lists, nqb, topk] int32 (device), lists == H (per-q-head lists, q head h
 *       served by kv head h / (H/Hkv)) or lists == Hkv (shared lists); entries outside
 *       [0, C) with C = T / chunk count as absent;
 *     k_host/v_host: the host-tier history, T tokens, batch stride host_bstride;
 *   out (device):
 *     chunk_of [B, Hkv, max_slots] int32: slot s of kv head j holds history chunk
 *       chunk_of[b, j, s]; the union of the chunks named by the lists served by kv head
 *       j, ascending, then -1;
 *     count [B, Hkv] int32: slots in use;
 *     idx_staged [B, lists, nqb, topk] int32: every entry replaced by its chunk's slot
 *       (absent entries -1), entry order kept;
 *     k_stage/v_stage [B, max_slots * chunk, Hkv, d] bf16 with batch stride
 *       stage_bstride: rows [s*chunk, (s+1)*chunk) of kv head j = rows of history chunk
 *       chunk_of[b, j, s] of kv head j (bit-exact copy); rows of unused slots untouched.
 *   Then hga_fwd / hga_bwd_active (or the _shared forms) with k_hist = k_stage,
 *   hist_bstride = stage_bstride, T = max_slots * chunk and idx = idx_staged reproduce
 *   the calls on the full history with idx.  Two launches on `stream` (plan, gather).
 * Checks: lists % Hkv == 0, T % chunk == 0, chunk % 64 == 0, 1 <= topk <= 64,
 *   C <= S2A_STAGE_MAX_CHUNKS (UNSUPPORTED above), and max_slots >= min(C, (lists/Hkv) *
 *   nqb * topk), the most chunks one kv head's lists can name, so that the union always
 *   fits; k_host/v_host pinned (only read when C > 0).
 * ------------------------------------------------------------------------------------ */
#define S2A_STAGE_MAX_CHUNKS 32768
#define S2A_STAGE_MAX_SLOTS 16384
int hga_detach_segment(const void* k_seg, const void* v_seg, long long seg_bstride, void* k_host, void* v_host,
                       long long host_bstride, float* summ, long long summ_bstride, int B, int S, int Hkv, int d,
                       int T, int chunk, void* stream);
int hga_stage_selected(const int32_t* idx, int lists, int nqb, int topk, const void* k_host, const void* v_host,
                       long long host_bstride, int T, int32_t* chunk_of, int32_t* count, int32_t* idx_staged,
                       void* k_stage, void* v_stage, long long stage_bstride, int max_slots, int B, int Hkv,
                       int d, int chunk, void* stream);

/* hga_stage_update: hga_stage_selected with the staging history kept as a cache across
 * calls, so that consecutive segments, whose lists name mostly the same chunks, copy only
 * the chunks the staging does not hold yet.
 *   chunk_of [B, Hkv, max_slots] int32 (device, in/out): on entry the chunk each slot of
 *     k_stage/v_stage holds, -1 for a free slot; the table a previous call on the same
 *     staging buffers and the same host history left (whose rows [0, T) must not have
 *     changed since), or all -1 for empty buffers.  Entries must be distinct.  On exit:
 *     slots whose chunk is named by the lists keep it; the other slots are freed; the named
 *     chunks not held take the free slots, ascending chunks into ascending slots; the rest
 *     of the free slots are -1.
 *   count [B, Hkv]: slots in use (distinct named chunks); copied [B, Hkv]: chunks copied
 *   from host memory by this call; copy_list [B, Hkv, max_slots] int32: scratch (the
 *   copies, slot << 16 | chunk), contents undefined on exit.
 *   idx_staged, k_stage, v_stage: as in hga_stage_selected (rows of kept slots are not
 *   written again).  The attention calls on the staging history give the same results,
 *   bit for bit, as on the full history.
 * Checks: those of hga_stage_selected, and max_slots <= S2A_STAGE_MAX_SLOTS (UNSUPPORTED
 * above). */
int hga_stage_update(const int32_t* idx, int lists, int nqb, int topk, const void* k_host, const void* v_host,
                     long long host_bstride, int T, int32_t* chunk_of, int32_t* count, int32_t* copied,
                     int32_t* copy_list, int32_t* idx_staged, void* k_stage, void* v_stage, long long stage_bstride,
                     int max_slots, int B, int Hkv, int d, int chunk, void* stream);

/* ------------------------------------------------------------------------------------
 * HGA generation step (same page: the method also serves retrieval and generation).  The
 * last nq tokens of an active segment of Sa tokens: query i (q[b, i, h, :]) sits at
 * segment position t = Sa - nq + i and attends, under ONE softmax with logit scale
 * `scale`, to
 *   (i)  active keys u <= t of k_act/v_act (Sa tokens), and
 *   (ii) every token of each chunk listed in idx[b, h, :] (entries >= 0; -1 = none), the
 *        chunk list of the query block the tokens belong to, chosen by the caller.
 *   q [B,nq,H,d] bf16; k_act/v_act bf16 with element (b,u,j,e) at
 *   k_act[b*act_bstride + (u*Hkv+j)*d + e] (u < Sa); k_hist/v_hist likewise with
 *   hist_bstride (T tokens); idx [B,H,topk] int32, valid entries < T/chunk.
 *   out: o [B,nq,H,d] bf16, lse [B,H,nq] float32.
 *   workspace: at least hga_decode_workspace_bytes(...) bytes (float32 partial results
 *   of the key splits), owned by the caller, contents undefined on entry and on exit.
 * Checks: 1 <= nq <= 32 (UNSUPPORTED above), nq <= Sa, T % chunk == 0, chunk % 64 == 0,
 * 1 <= topk <= 64.  Two launches on `stream` (split partials, then their merge).
 * ------------------------------------------------------------------------------------ */
size_t hga_decode_workspace_bytes(int B, int nq, int Sa, int H, int d, int chunk, int topk);
int hga_decode(const void* q, const void* k_act, const void* v_act, long long act_bstride,
               const void* k_hist, const void* v_hist, long long hist_bstride, const int32_t* idx,
               void* o, float* lse, void* workspace, size_t workspace_bytes,
               int B, int nq, int Sa, int H, int Hkv, int d, int T, int chunk, int topk, float scale,
               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* S2A_H */
