// Host-side hand-off of a decoded utterance: incremental un-delay, chunked emission and
// the repeated-code stop guard (include/hta.h, hta_stream_*).
//
// Reference: FlashRT "Higgs Audio v3 TTS-4B" page, section 4 (a streaming generator whose
// output equals the one-shot output), section 5 (greedy generation applies the delay
// pattern and un-delays the codes before the codec) and its Performance section (a
// deterministic repeated-code stop guard ends pathological runs that never emit EOC, before
// the generation cap).  The page gives no guard rule; the one taken here watches complete
// frames and fires at the first frame that ends a window of `window` frames repeating with
// a period of at most `max_period` frames.
#include <cstring>
#include <new>
#include <vector>

#include "hta_internal.h"

struct hta_stream {
  int C, bos, eos, chunk, window, max_period;
  std::vector<int32_t> steps;   // every step's C codes pushed so far
  std::vector<int32_t> frames;  // every complete un-delayed frame [n][C]
  long eoc = -1;                // first step at which codebook 0 holds EOS
  long emitted = 0;             // frames handed to the caller
  int status = HTA_STREAM_RUNNING;
};

namespace {

// Frame f repeats the frame p before it.
bool same_frame(const hta_stream& s, long f, int p) {
  return std::memcmp(&s.frames[(size_t)f * s.C], &s.frames[(size_t)(f - p) * s.C], sizeof(int32_t) * s.C) == 0;
}

// The last `window` frames (ending at frame f) repeat with some period p <= max_period.
bool guard_fires(const hta_stream& s, long f) {
  if (s.window <= 0 || f + 1 < s.window) return false;
  const long first = f - s.window + 1;
  for (int p = 1; p <= s.max_period && p < s.window; ++p) {
    bool periodic = true;
    for (long g = first + p; g <= f && periodic; ++g) periodic = same_frame(s, g, p);
    if (periodic) return true;
  }
  return false;
}

// Take the frames that became complete with the steps pushed so far.
void complete_frames(hta_stream& s) {
  const long n_steps = (long)(s.steps.size() / s.C);
  while (s.status == HTA_STREAM_RUNNING) {
    const long f = (long)(s.frames.size() / s.C);
    if (s.eoc >= 0 && f >= s.eoc) {  // every frame before EOC is complete once step eoc + C - 2 is in
      s.status = HTA_STREAM_DONE;
      break;
    }
    if (f + s.C - 1 >= n_steps) break;  // frame f needs step f + C - 1
    for (int k = 0; k < s.C; ++k) s.frames.push_back(s.steps[(size_t)(f + k) * s.C + k]);
    if (guard_fires(s, f)) s.status = HTA_STREAM_STOPPED;
  }
}

}  // namespace

extern "C" {

int hta_stream_create(int n_codebooks, int bos_id, int eos_id, int chunk_frames, int guard_window,
                      int guard_max_period, hta_stream** out) {
  if (!out) return HTA_E_ARG;
  *out = nullptr;
  if (n_codebooks < 1 || n_codebooks > 64 || chunk_frames < 1 || guard_window < 0 || guard_max_period < 0)
    return HTA_E_ARG;
  hta_stream* s = new (std::nothrow) hta_stream();
  if (!s) return HTA_E_ARG;
  s->C = n_codebooks;
  s->bos = bos_id;
  s->eos = eos_id;
  s->chunk = chunk_frames;
  s->window = guard_window;
  s->max_period = guard_max_period;
  *out = s;
  return HTA_OK;
}

int hta_stream_push(hta_stream* s, const int32_t* step_codes, int n_steps, int32_t* frames_out, int max_frames,
                    int* n_frames, int* status) {
  if (!s || n_steps < 0 || (n_steps > 0 && !step_codes) || max_frames < 0 || (max_frames > 0 && !frames_out) ||
      !n_frames)
    return HTA_E_ARG;
  *n_frames = 0;
  // steps after the utterance ended (done or stopped) are ignored
  for (int i = 0; i < n_steps && s->status == HTA_STREAM_RUNNING; ++i) {
    const long t = (long)(s->steps.size() / s->C);
    s->steps.insert(s->steps.end(), step_codes + (size_t)i * s->C, step_codes + (size_t)(i + 1) * s->C);
    if (s->eoc < 0 && step_codes[(size_t)i * s->C] == s->eos) s->eoc = t;
    complete_frames(*s);
  }
  // whole chunks while running; everything once the utterance has ended
  const long ready = (long)(s->frames.size() / s->C) - s->emitted;
  long give = s->status == HTA_STREAM_RUNNING ? ready / s->chunk * s->chunk : ready;
  if (give > max_frames) give = s->status == HTA_STREAM_RUNNING ? (long)max_frames / s->chunk * s->chunk : max_frames;
  if (give > 0)
    std::memcpy(frames_out, &s->frames[(size_t)s->emitted * s->C], sizeof(int32_t) * (size_t)give * s->C);
  s->emitted += give;
  *n_frames = (int)give;
  if (status) *status = s->status;
  return HTA_OK;
}

int hta_stream_finish(hta_stream* s, int32_t* frames_out, int max_frames, int* n_frames) {
  if (!s || max_frames < 0 || (max_frames > 0 && !frames_out) || !n_frames) return HTA_E_ARG;
  if (s->status == HTA_STREAM_RUNNING) s->status = HTA_STREAM_CAPPED;
  int st = 0;
  return hta_stream_push(s, nullptr, 0, frames_out, max_frames, n_frames, &st);
}

void hta_stream_destroy(hta_stream* s) { delete s; }

}  // extern "C"
