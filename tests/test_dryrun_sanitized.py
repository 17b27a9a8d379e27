"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer,
with no GPU: tests/dryrun_check.cpp (gdn_api.cpp compiled into it with the host
sanitizers, built by __graft_entry__.build()) drives dry-run handles and
gdn_forward_noalloc's dry run through valid calls and every rejection path; any
sanitizer report or leak fails the run."""
import os
import subprocess

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dryrun_check")


def test_dry_run_validation_is_sanitizer_clean():
    assert os.path.exists(EXE), "tests/dryrun_check is not built (run __graft_entry__.build())"
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout)
    print(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert r.stdout.strip().splitlines()[-1] == "dry-run check ok"
