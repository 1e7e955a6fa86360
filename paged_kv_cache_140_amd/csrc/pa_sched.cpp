// Chunked prefill under a per-step token budget: which prompts' chunks ride
// along with a step's decode tokens ([ttlab]
// "llm-kv-cache-02-serving-engine-kv", section "3. 연속 배칭: 빈 자리를 걸음마다
// 채우기", part "새 문제: 긴 프리필이 디코드를 멈춘다").  A long prompt
// prefilled in one step stalls every running request's next token; cut into
// chunks under a cap on the tokens a step processes, it shares each step
// with the decodes.  The cap counts every token: each running decode takes
// one and is never postponed, then the waiting prompts, in arrival order,
// take chunks of their remaining prompt tokens until the cap is spent.  The
// result is a pa_mixed_batch chunk list.
#include "pa_host.h"

extern "C" int pa_plan_step(int32_t budget, int32_t n_decode, const pa_prompt_state* prompts, int32_t n_prompts,
                            int32_t max_chunks, pa_chunk_plan* out, int32_t* n_out) {
  using namespace pa;
  if (n_decode < 0 || n_prompts < 0 || max_chunks < 0 || !n_out || (n_prompts > 0 && !prompts) ||
      (max_chunks > 0 && !out))
    return fail(PA_EINVAL, "pa_plan_step: bad argument");
  for (int32_t i = 0; i < n_prompts; ++i)
    if (prompts[i].prompt_len < 0 || prompts[i].computed < 0 || prompts[i].computed > prompts[i].prompt_len)
      return fail(PA_EINVAL, "pa_plan_step: prompt " + std::to_string(i) + " has computed outside [0, prompt_len]");
  int64_t left = static_cast<int64_t>(budget) - n_decode;
  int32_t n = 0;
  for (int32_t i = 0; i < n_prompts && left > 0 && n < max_chunks; ++i) {
    const int32_t rest = prompts[i].prompt_len - prompts[i].computed;
    if (rest <= 0) continue;
    const int32_t t = static_cast<int32_t>(std::min<int64_t>(rest, left));
    out[n++] = pa_chunk_plan{i, prompts[i].computed, t};
    left -= t;
  }
  *n_out = n;
  return PA_OK;
}
